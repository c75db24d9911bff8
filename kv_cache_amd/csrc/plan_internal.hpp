// Host helpers shared by the planner and the launch code.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

#include "decode_attn.h"

namespace da {

// FNV-1a over the plan bytes that follow the key field.  The plan is a
// padding-free POD (int32/float fields, then 8-byte aligned uint64 fields).
inline uint64_t plan_hash(const da_plan& p) {
  const unsigned char* b = reinterpret_cast<const unsigned char*>(&p);
  const size_t begin = offsetof(da_plan, problem);
  const size_t end = offsetof(da_plan, reserved);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = begin; i < end; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

inline bool plan_intact(const da_plan* p) { return p && p->key == plan_hash(*p); }

// Workspace layout: u [rows,S,D] f32, m [rows,S] f32, l [rows,S] f32 with
// rows = B*C*H_q ordered (b, i, h_q), then (at a 256-byte boundary) one uint32
// arrival counter per (b, h_kv), then (at a 256-byte boundary) the partition
// header [W, L, B, 0, P_0 .. P_B] that every run writes for the combine.
inline uint64_t states_bytes_raw(int64_t rows, int64_t S, int64_t Dv) {
  return (uint64_t)(rows * S * (Dv + 2) * 4);
}
inline uint64_t round_up_256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }
inline int64_t output_rows(const da_problem& p) {
  return (int64_t)p.batch * p.num_queries * p.num_q_heads;
}
inline uint64_t states_bytes(const da_plan& p) {
  return round_up_256(states_bytes_raw(output_rows(p.problem), p.num_splits, p.problem.head_dim_v));
}
inline uint64_t counters_bytes(int64_t groups) { return round_up_256((uint64_t)(groups * 4)); }
inline uint64_t partition_header_bytes(int64_t batch) { return round_up_256((uint64_t)((batch + 5) * 4)); }
inline uint64_t workspace_bytes_for(int64_t rows, int64_t groups, int64_t batch, int64_t S, int64_t Dv) {
  return round_up_256(states_bytes_raw(rows, S, Dv)) + counters_bytes(groups) + partition_header_bytes(batch);
}
// Byte offset of the partition header in the workspace.
inline uint64_t partition_header_offset(const da_plan& p) {
  return states_bytes(p) + counters_bytes((int64_t)p.problem.batch * p.problem.num_kv_heads);
}

// Element size in bytes of one K/V row element as stored in k/v.
inline int kv_elem_bytes(int kv_format) {
  return kv_format == DA_KV_F32 ? 4 : kv_format == DA_KV_BF16 ? 2 : 1;
}

// Queries the current device: CU count and whether it is gfx950.  Returns
// false if the HIP runtime cannot answer.
bool current_device_info(int* device, int* num_cus, bool* is_gfx950);

// Per-device cached gfx950 check used by the launch entry points.
bool current_device_is_gfx950();

}  // namespace da
