// Internal declarations shared by the host lowering (lower.cpp) and the HIP runtime
// (runtime.hip).  Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mk.h"

namespace mk {

// Canonical buffer-table indices (append-only order: per-step inputs, weights and
// caches, then the step's activations in emission order, then logits).
struct BufIdx {
  int L = 0;
  bool unfused = false;  // five more activation buffers per layer group (extra())
  uint32_t tokens() const { return 0; }
  uint32_t positions() const { return 1; }
  uint32_t embedding() const { return 2; }
  uint32_t layer(int l, int which) const { return 3u + 8u * l + which; }  // 0..7
  uint32_t final_norm() const { return 3u + 8u * L; }
  uint32_t w_lm() const { return 4u + 8u * L; }
  uint32_t x0() const { return 5u + 8u * L; }
  // which: 0 qkv_out, 1 q_rot, 2 partials, 3 att, 4 h, 5 gu, 6 x_out
  uint32_t act(int l, int which) const { return 6u + 8u * L + 7u * l + which; }
  uint32_t logits() const { return 6u + 15u * L; }
  // Graphs lowered without epilogue fusion only, appended after the logits.  which:
  // 0 normed attention input, 1 o-projection output, 2 normed MLP input, 3 down-
  // projection output; l = L with which 0: the normed input of the lm_head.
  uint32_t extra(int l, int which) const { return 7u + 15u * L + 4u * l + which; }
  uint32_t count() const { return 7u + 15u * L + (unfused ? 4u * L + 1u : 0u); }
};


enum { W_ATTN_NORM = 0, W_QKV, W_O, W_MLP_NORM, W_GATE_UP, W_DOWN, KCACHE, VCACHE };
constexpr uint16_t kNone = 0xFFFF;

// Blob header: 64 bytes in front of the task array on the device.
struct BlobHeader {
  uint32_t magic;  // 'MKG1'
  uint32_t abi_version;
  uint32_t n_tasks;
  uint32_t n_edges;
  uint32_t n_buffers;
  float rms_eps;
  float rope_theta;
  int32_t kv_chunk;
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, batch, intermediate, vocab, kv_capacity;
};
static_assert(sizeof(BlobHeader) == 64, "blob header must be 64 bytes");

// A contiguous run of tasks of one op in emission order (NOPs excluded): the unit of
// one launch in the per-op baseline.
struct OpRange {
  uint32_t first;
  uint32_t count;
  uint16_t op_id;
};

struct Lowered {
  mk_model_cfg cfg{};
  std::vector<int32_t> kv_len;
  BufIdx bi;
  BlobHeader header{};
  std::vector<mk_task_t> tasks;
  std::vector<uint32_t> edges;
  std::vector<OpRange> ops;
  std::vector<uint64_t> scratch_off;    // per buffer; UINT64_MAX if not scratch
  std::vector<uint64_t> scratch_size;
  uint64_t scratch_total = 0;
  uint64_t kv_layer_bytes = 0;
  uint32_t n_levels = 0;
};

int validate_cfg(const mk_model_cfg* cfg);
int lower(const mk_model_cfg* cfg, Lowered& out);

// Static schedule: the non-NOP tasks split into one list per workgroup, each list in
// increasing task order (so the topological-order deadlock argument holds per list).
// Built by simulating list scheduling in emission order with a byte-count cost model:
// each task goes to the workgroup that can start it earliest.  NOP joins get no
// workgroup: their parents count on the join's counter and its children poll it.
struct Schedule {
  std::vector<uint32_t> order;    // task indices, grouped by workgroup
  std::vector<uint32_t> offsets;  // [workers + 1]
  double est_us = 0;              // simulated step time (diagnostic)
};
void build_schedule(const Lowered& L, uint32_t workers, Schedule& out);

// Level-synchronous lists: the non-NOP tasks grouped by their level in the DAG.
struct Levels {
  std::vector<uint32_t> tasks;    // task indices, grouped by level, ascending within one
  std::vector<uint32_t> offsets;  // [levels + 1]
};
void build_levels(const Lowered& L, Levels& out);

int set_error(int code, const std::string& msg);
int set_error(int code, const char* msg);  // allocates nothing

}  // namespace mk

struct mk_lowered {
  mk::Lowered low;
  mk::Schedule sched;
  mk::Levels levels;
};
