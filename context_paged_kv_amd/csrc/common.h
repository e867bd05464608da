// Internal helpers shared by the library's translation units.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "dcpkv.h"

namespace dcpkv {

// Record a formatted message for dcpkv_last_error() and return `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxShards = 64;    // N destination pools / DCP shards per call
constexpr int kMaxSources = 64;   // N_cp layer-split sources per call
constexpr int kMaxLayers = 256;   // layers per reshard call

}  // namespace dcpkv
