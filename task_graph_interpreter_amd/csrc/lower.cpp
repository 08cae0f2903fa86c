// Host lowering: one decode step -> 64-byte task descriptors + CSR dependents array.
//
// Follows "Mega kernel initial" (1y33.com): the lowering section (each matmul fans out
// into one GEMV task per output-column tile; attention becomes one ATTENTION_PARTIAL per
// (sequence, KV-head group, KV chunk) and a combine; RMSNorm, residual and SiLU*mul are
// flags of the consuming GEMV; the final norm is fused into the lm_head GEMV), the
// descriptor section (uint16 buffer indices, per-op reserved scalars, flag bits) and the
// edge section (every task records which earlier tasks wrote the column ranges it reads;
// parents are inverted into one flat dependents array; emission order is topological).
//
// Conventions where the page is silent (same as the oracle lowering):
//  * reads/writes are (row range) x (column range) rectangles of a buffer, rows being
//    batch rows, so batch > 1 tracks per-sequence attention tasks exactly;
//  * every op output is a fresh buffer (single assignment), so only read-after-write
//    edges exist;
//  * one combine per (sequence, KV-head group); one APPEND per (sequence, group) that
//    rotates the group's q heads and its k head and appends k and v;
//  * join NOPs: for an op with >= 2 tasks whose tasks share >= 2 parents, one NOP with
//    those parents is emitted just before the op and replaces them in every task's
//    parent list (a T x T boundary becomes 2 T edges);
//  * the step is first written as a list of ops the way the page's graph API builds it,
//    with no fusion: every RMSNorm its own op, each residual add carried by the next
//    RMSNorm (FUSED_RESIDUAL, flags paragraph).  The epilogue-fusion pass the graph-API
//    section names as future work then folds each residual add into the matmul that
//    produced the summand and each RMSNorm read only by matmuls into those matmuls,
//    which gives the hand-fused decoder of that section; MK_LOWER_UNFUSED skips it.
//    RMSNORM (OpId 3) is one task per batch row; with MK_LOWER_SAMPLE one SAMPLE task
//    (OpId 6) per row follows the lm_head.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>

#include "internal.h"

namespace mk {

namespace {

struct Rect {
  uint32_t buf;
  int64_t r0, r1, c0, c1;
};

struct Writer {
  int64_t r0, r1, c0, c1;
  uint32_t task;
};

struct PendingTask {
  mk_task_t d;
  Rect reads[3];
  int n_reads;
  Rect writes[2];
  int n_writes;
};

inline bool overlap(const Writer& w, const Rect& r) {
  return w.r0 < r.r1 && r.r0 < w.r1 && w.c0 < r.c1 && r.c0 < w.c1;
}

mk_task_t blank() {
  mk_task_t t;
  std::memset(&t, 0, sizeof(t));
  t.in_buf[0] = t.in_buf[1] = t.in_buf[2] = kNone;
  t.out_buf = kNone;
  return t;
}

class Builder {
 public:
  explicit Builder(Lowered& L) : L_(L), writers_(L.bi.count()) {}

  // Adds one op's tasks: computes parents from the writer index, applies the join
  // rule, appends descriptors and records their writes.
  void emit(std::vector<PendingTask>& op) {
    std::vector<std::vector<uint32_t>> par(op.size());
    for (size_t i = 0; i < op.size(); ++i) {
      std::vector<uint32_t>& p = par[i];
      for (int r = 0; r < op[i].n_reads; ++r) {
        const Rect& rd = op[i].reads[r];
        for (const Writer& w : writers_[rd.buf])
          if (overlap(w, rd)) p.push_back(w.task);
      }
      std::sort(p.begin(), p.end());
      p.erase(std::unique(p.begin(), p.end()), p.end());
    }
    if (L_.cfg.join_nodes && op.size() >= 2) {
      std::vector<uint32_t> common = par[0];
      for (size_t i = 1; i < op.size() && !common.empty(); ++i) {
        std::vector<uint32_t> tmp;
        std::set_intersection(common.begin(), common.end(), par[i].begin(), par[i].end(),
                              std::back_inserter(tmp));
        common.swap(tmp);
      }
      if (common.size() >= 2) {
        uint32_t nop = (uint32_t)L_.tasks.size();
        L_.tasks.push_back(blank());  // op_id NOP = 0
        parents_.push_back(common);
        for (auto& p : par) {
          std::vector<uint32_t> rest;
          std::set_difference(p.begin(), p.end(), common.begin(), common.end(), std::back_inserter(rest));
          rest.push_back(nop);  // the NOP is newer than every other parent
          p.swap(rest);
        }
      }
    }
    uint32_t first = (uint32_t)L_.tasks.size();
    for (size_t i = 0; i < op.size(); ++i) {
      uint32_t idx = (uint32_t)L_.tasks.size();
      L_.tasks.push_back(op[i].d);
      parents_.push_back(std::move(par[i]));
      for (int k = 0; k < op[i].n_writes; ++k) {
        const Rect& w = op[i].writes[k];
        writers_[w.buf].push_back(Writer{w.r0, w.r1, w.c0, w.c1, idx});
      }
    }
    if (!op.empty()) L_.ops.push_back(OpRange{first, (uint32_t)op.size(), op[0].d.op_id});
  }

  // Inverts parents into the CSR dependents array and fills the dependency fields.
  void finish() {
    const size_t n = L_.tasks.size();
    std::vector<uint32_t> outdeg(n, 0);
    for (size_t t = 0; t < n; ++t)
      for (uint32_t p : parents_[t]) ++outdeg[p];
    uint64_t off = 0;
    std::vector<uint64_t> cursor(n);
    for (size_t t = 0; t < n; ++t) {
      L_.tasks[t].dependents_offset = (uint32_t)off;
      L_.tasks[t].num_dependents = (int32_t)outdeg[t];
      L_.tasks[t].remaining_deps = (int32_t)parents_[t].size();
      cursor[t] = off;
      off += outdeg[t];
    }
    L_.edges.assign(off, 0);
    // Children are visited in ascending order, so every dependents list is ascending.
    for (size_t t = 0; t < n; ++t)
      for (uint32_t p : parents_[t]) L_.edges[cursor[p]++] = (uint32_t)t;
    std::vector<uint32_t> level(n, 0);
    uint32_t maxl = 0;
    for (size_t t = 0; t < n; ++t) {
      uint32_t lv = 0;
      for (uint32_t p : parents_[t]) lv = std::max(lv, level[p] + 1);
      level[t] = lv;
      maxl = std::max(maxl, lv);
    }
    L_.n_levels = n ? maxl + 1 : 0;
  }

 private:
  Lowered& L_;
  std::vector<std::vector<Writer>> writers_;
  std::vector<std::vector<uint32_t>> parents_;
};

// One op of the step before its fan-out into tasks.  MATMUL: out = x W^T with the
// epilogue flags gamma (RMS_NORM_INPUT), residual (ADD_RESIDUAL) and silu (SILU_MUL).
// NORM: out = rmsnorm(x [+ residual]) * gamma, also writing the sum to out2 when there
// is a residual (FUSED_RESIDUAL).  ATTN: layer `layer` from its qkv input x.  EMBED:
// x0 from the tokens.  SAMPLE: greedy token of each row of x into out (tokens), the
// row's position (out2) advanced.
enum class OpKind { EMBED, NORM, MATMUL, ATTN, SAMPLE };

struct Op {
  OpKind kind;
  uint32_t out, x = kNone, w = kNone, gamma = kNone, residual = kNone, out2 = kNone;
  bool silu = false;
  int64_t K = 0, N = 0;
  int layer = -1;
  bool dead = false;
};

// The decode step written with the graph API and no fusion.
std::vector<Op> decoder_program(const mk_model_cfg& c, const BufIdx& bi) {
  const int64_t H = c.hidden, I = c.intermediate, V = c.vocab, L = c.n_layers;
  const int64_t qkv_cols = (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim,
                qcols = (int64_t)c.n_q_heads * c.head_dim;
  std::vector<Op> ops;
  auto add = [&](Op o) { ops.push_back(o); };
  {
    Op e{OpKind::EMBED, bi.x0()};
    e.x = bi.tokens();
    e.w = bi.embedding();
    add(e);
  }
  uint32_t x_in = bi.x0();
  for (int l = 0; l < L; ++l) {
    Op n1{OpKind::NORM, bi.extra(l, 0)};
    n1.gamma = bi.layer(l, W_ATTN_NORM);
    n1.N = H;
    if (l == 0) {
      n1.x = bi.x0();
    } else {  // the previous layer's residual add rides on this norm
      n1.x = bi.extra(l - 1, 3);
      n1.residual = bi.act(l - 1, 4);
      n1.out2 = x_in;
    }
    add(n1);
    Op q{OpKind::MATMUL, bi.act(l, 0)};
    q.x = bi.extra(l, 0), q.w = bi.layer(l, W_QKV), q.K = H, q.N = qkv_cols;
    add(q);
    Op a{OpKind::ATTN, bi.act(l, 3)};
    a.x = bi.act(l, 0), a.layer = l;
    add(a);
    Op o{OpKind::MATMUL, bi.extra(l, 1)};
    o.x = bi.act(l, 3), o.w = bi.layer(l, W_O), o.K = qcols, o.N = H;
    add(o);
    Op n2{OpKind::NORM, bi.extra(l, 2)};
    n2.x = bi.extra(l, 1), n2.gamma = bi.layer(l, W_MLP_NORM), n2.residual = x_in, n2.out2 = bi.act(l, 4), n2.N = H;
    add(n2);
    Op g{OpKind::MATMUL, bi.act(l, 5)};
    g.x = bi.extra(l, 2), g.w = bi.layer(l, W_GATE_UP), g.silu = true, g.K = H, g.N = I;
    add(g);
    Op d{OpKind::MATMUL, bi.extra(l, 3)};
    d.x = bi.act(l, 5), d.w = bi.layer(l, W_DOWN), d.K = I, d.N = H;
    add(d);
    x_in = bi.act(l, 6);
  }
  Op nf{OpKind::NORM, bi.extra((int)L, 0)};
  nf.x = bi.extra((int)L - 1, 3), nf.gamma = bi.final_norm(), nf.residual = bi.act((int)L - 1, 4), nf.out2 = x_in;
  nf.N = H;
  add(nf);
  Op lm{OpKind::MATMUL, bi.logits()};
  lm.x = bi.extra((int)L, 0), lm.w = bi.w_lm(), lm.K = H, lm.N = V;
  add(lm);
  return ops;
}

// The automatic epilogue-fusion pass.
//  1. A norm with a residual whose input is written by a matmul with no epilogue and
//     read by nothing else: the matmul adds the residual itself (ADD_RESIDUAL) and
//     writes the sum; the norm then reads the sum with no residual.
//  2. A norm with no residual whose every reader is a matmul taking it as its input,
//     with neither an input norm nor a residual (one gamma/residual slot per
//     descriptor): each reader reads the norm's input with RMS_NORM_INPUT, and the
//     norm is dropped.
void fuse_epilogues(std::vector<Op>& ops) {
  auto readers = [&](uint32_t buf) {
    std::vector<size_t> r;
    for (size_t i = 0; i < ops.size(); ++i)
      if (!ops[i].dead && (ops[i].x == buf || ops[i].residual == buf)) r.push_back(i);
    return r;
  };
  auto writers = [&](uint32_t buf) {
    std::vector<size_t> r;
    for (size_t i = 0; i < ops.size(); ++i)
      if (!ops[i].dead && (ops[i].out == buf || ops[i].out2 == buf)) r.push_back(i);
    return r;
  };
  for (size_t i = 0; i < ops.size(); ++i) {
    Op& n = ops[i];
    if (n.kind != OpKind::NORM || n.residual == kNone) continue;
    const std::vector<size_t> wr = writers(n.x), rd = readers(n.x);
    if (wr.size() != 1 || rd.size() != 1 || rd[0] != i) continue;
    Op& m = ops[wr[0]];
    if (m.kind != OpKind::MATMUL || m.gamma != kNone || m.residual != kNone || m.silu) continue;
    m.residual = n.residual;
    m.out = n.out2;
    n.x = n.out2;
    n.residual = kNone;
    n.out2 = kNone;
  }
  for (size_t i = 0; i < ops.size(); ++i) {
    Op& n = ops[i];
    if (n.dead || n.kind != OpKind::NORM || n.residual != kNone) continue;
    const std::vector<size_t> rd = readers(n.out);
    bool ok = !rd.empty();
    for (size_t r : rd) {
      const Op& m = ops[r];
      ok = ok && m.kind == OpKind::MATMUL && m.x == n.out && m.gamma == kNone && m.residual == kNone;
    }
    if (!ok) continue;
    for (size_t r : rd) {
      ops[r].x = n.x;
      ops[r].gamma = n.gamma;
    }
    n.dead = true;
  }
  ops.erase(std::remove_if(ops.begin(), ops.end(), [](const Op& o) { return o.dead; }), ops.end());
}

void tile_range(int64_t N, int64_t T, int64_t i, bool mfma, int64_t& c0, int64_t& c1) {
  if (mfma) {
    int64_t n16 = N / 16;
    c0 = 16 * (i * n16 / T);
    c1 = 16 * ((i + 1) * n16 / T);
  } else {
    c0 = i * N / T;
    c1 = (i + 1) * N / T;
  }
}

}  // namespace

int validate_cfg(const mk_model_cfg* c) {
  if (!c) return set_error(MK_ERR_INVALID, "cfg is NULL");
  if (c->abi_version != MK_ABI_VERSION || c->struct_size != sizeof(mk_model_cfg))
    return set_error(MK_ERR_ABI, "mk_model_cfg abi_version/struct_size mismatch");
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->intermediate < 1 || c->vocab < 1 || c->batch < 1)
    return set_error(MK_ERR_INVALID, "model dimensions must be positive");
  if (c->n_q_heads % c->n_kv_heads) return set_error(MK_ERR_INVALID, "n_q_heads % n_kv_heads != 0");
  if (c->head_dim % 2) return set_error(MK_ERR_INVALID, "head_dim must be even (rotate-half RoPE)");
  if (c->weight_dtype != MK_DTYPE_F32 && c->weight_dtype != MK_DTYPE_BF16)
    return set_error(MK_ERR_INVALID, "weight_dtype must be MK_DTYPE_F32 or MK_DTYPE_BF16");
  if (c->kv_dtype != MK_DTYPE_F32 && c->kv_dtype != MK_DTYPE_BF16)
    return set_error(MK_ERR_INVALID, "kv_dtype must be MK_DTYPE_F32 or MK_DTYPE_BF16");
  if (c->gemv_config < 0 || c->gemv_config > 2) return set_error(MK_ERR_INVALID, "gemv_config out of range");
  if ((c->gemv_config == MK_GEMV_F32) != (c->weight_dtype == MK_DTYPE_F32))
    return set_error(MK_ERR_INVALID, "gemv_config 0 is the fp32-weight variant; 1 and 2 need bf16 weights");
  if (c->kv_chunk < 1 || c->kv_capacity < 1) return set_error(MK_ERR_INVALID, "kv_chunk/kv_capacity must be >= 1");
  if (!c->kv_len) return set_error(MK_ERR_INVALID, "kv_len is NULL");
  for (int b = 0; b < c->batch; ++b)
    if (c->kv_len[b] < 1 || c->kv_len[b] > c->kv_capacity)
      return set_error(MK_ERR_INVALID, "kv_len[b] must be in [1, kv_capacity]");
  const int64_t qkv = (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
  const int64_t Ns[4] = {qkv, c->hidden, c->intermediate, c->vocab};
  for (int64_t N : Ns) {
    if (c->gemv_config == MK_GEMV_BF16_MFMA) {
      if (N % 16) return set_error(MK_ERR_INVALID, "MFMA GEMV needs every output width % 16 == 0");
      if (c->gemv_tiles < 1 || c->gemv_tiles > N / 16)
        return set_error(MK_ERR_INVALID, "gemv_tiles must be in [1, N/16] for the MFMA GEMV");
    } else if (c->gemv_tiles < 1 || c->gemv_tiles > N) {
      return set_error(MK_ERR_INVALID, "gemv_tiles must be in [1, N] for every matmul");
    }
  }
  if (c->options & ~(MK_LOWER_UNFUSED | MK_LOWER_SAMPLE | MK_LOWER_PACKED_WEIGHTS))
    return set_error(MK_ERR_INVALID, "unknown bit in options");
  if ((c->options & MK_LOWER_PACKED_WEIGHTS) && c->gemv_config != MK_GEMV_BF16_MFMA)
    return set_error(MK_ERR_INVALID, "MK_LOWER_PACKED_WEIGHTS needs the MFMA GEMV (gemv_config 2)");
  if (7ll + 15ll * c->n_layers + ((c->options & MK_LOWER_UNFUSED) ? 4ll * c->n_layers + 1 : 0) > 0xFFFF)
    return set_error(MK_ERR_INVALID, "more than 65535 buffers");
  // Limits of the device task bodies: GEMV rows are streamed in 16-byte pieces and an
  // input row is staged in the 148 KB LDS area; a KV row is read by a power-of-two
  // group of lanes, 16 bytes each.  The chunk length and the number of chunks have no
  // device limit (a partial keeps its running sums in registers, a combine folds
  // blocks of 16 chunks).
  const int64_t wes = c->weight_dtype == MK_DTYPE_F32 ? 4 : 2, kes = c->kv_dtype == MK_DTYPE_F32 ? 4 : 2;
  const int64_t Ks[3] = {c->hidden, (int64_t)c->n_q_heads * c->head_dim, c->intermediate};
  for (int64_t K : Ks) {
    if ((K * wes) % 16) return set_error(MK_ERR_INVALID, "GEMV inner dims must be multiples of 16 bytes");
    if (K > 32768) return set_error(MK_ERR_INVALID, "GEMV inner dim above 32768 (LDS staging)");
    if (c->gemv_config == MK_GEMV_BF16_MFMA && K % 256)
      return set_error(MK_ERR_INVALID, "the MFMA GEMV needs every inner dim % 256 == 0 (chunks of 8 x 32)");
    if (c->gemv_config == MK_GEMV_BF16_MFMA && (int64_t)c->batch * K * 4 >= (1ll << 32))
      return set_error(MK_ERR_INVALID, "the MFMA GEMV reads its fp32 input rows with 32-bit offsets: batch x K x 4 >= 4 GiB");
  }
  // The GEMV addresses a weight matrix with 32-bit byte offsets.
  const int64_t H = c->hidden;
  const int64_t wbytes[5] = {qkv * H, H * (int64_t)c->n_q_heads * c->head_dim, 2ll * c->intermediate * H,
                             H * (int64_t)c->intermediate, (int64_t)c->vocab * H};
  for (int64_t e : wbytes)
    if (e * wes >= (1ll << 32)) return set_error(MK_ERR_INVALID, "a weight matrix is 4 GiB or larger");
  // The attention partial addresses one (sequence, KV head)'s cache rows with 32-bit
  // byte offsets.
  if ((int64_t)c->kv_capacity * c->head_dim * kes >= (1ll << 32))
    return set_error(MK_ERR_INVALID, "one KV head's cache rows are 4 GiB or larger");
  const int64_t lpk = c->head_dim * kes / 16;
  if ((c->head_dim * kes) % 16 || lpk < 1 || lpk > 64 || (lpk & (lpk - 1)))
    return set_error(MK_ERR_INVALID, "head_dim * cache element size must be 16 * 2^j bytes, at most 1 KB");
  if (c->batch > (1 << 20) || c->kv_capacity > (1 << 30)) return set_error(MK_ERR_INVALID, "size too large");
  return MK_OK;
}

int lower(const mk_model_cfg* cfg, Lowered& L) {
  int rc = validate_cfg(cfg);
  if (rc) return rc;
  L = Lowered();
  L.cfg = *cfg;
  L.kv_len.assign(cfg->kv_len, cfg->kv_len + cfg->batch);
  L.cfg.kv_len = L.kv_len.data();
  L.bi.L = cfg->n_layers;
  L.bi.unfused = (cfg->options & MK_LOWER_UNFUSED) != 0;
  const BufIdx& bi = L.bi;

  const int64_t B = cfg->batch, H = cfg->hidden, hd = cfg->head_dim, Hq = cfg->n_q_heads,
                Hkv = cfg->n_kv_heads, I = cfg->intermediate, V = cfg->vocab, T = cfg->gemv_tiles;
  const int64_t grp = Hq / Hkv, qkv_cols = (Hq + 2 * Hkv) * hd, qcols = Hq * hd;
  const bool mfma = cfg->gemv_config == MK_GEMV_BF16_MFMA;
  const uint16_t kvc = (uint16_t)cfg->kv_dtype;

  std::vector<int64_t> chunks(B);
  std::vector<int64_t> slot_base(B * Hkv);
  int64_t n_slots = 0;
  for (int64_t b = 0; b < B; ++b) {
    chunks[b] = (L.kv_len[b] + cfg->kv_chunk - 1) / cfg->kv_chunk;
    for (int64_t g = 0; g < Hkv; ++g) {
      slot_base[b * Hkv + g] = n_slots;
      n_slots += chunks[b];
    }
  }

  // Scratch layout: activation buffers in index order, each 256-byte aligned.
  const uint32_t nb = bi.count();
  L.scratch_off.assign(nb, UINT64_MAX);
  L.scratch_size.assign(nb, 0);
  uint64_t off = 0;
  auto place = [&](uint32_t buf, uint64_t bytes) {
    L.scratch_off[buf] = off;
    L.scratch_size[buf] = bytes;
    off += (bytes + 255) & ~uint64_t(255);
  };
  place(bi.x0(), 4ull * B * H);
  for (int l = 0; l < cfg->n_layers; ++l) {
    place(bi.act(l, 0), 4ull * B * qkv_cols);
    place(bi.act(l, 1), 4ull * B * qcols);
    place(bi.act(l, 2), 4ull * n_slots * grp * (hd + 2));
    place(bi.act(l, 3), 4ull * B * qcols);
    place(bi.act(l, 4), 4ull * B * H);
    place(bi.act(l, 5), 4ull * B * I);
    place(bi.act(l, 6), 4ull * B * H);
  }
  if (bi.unfused) {
    for (int l = 0; l < cfg->n_layers; ++l)
      for (int j = 0; j < 4; ++j) place(bi.extra(l, j), 4ull * B * H);
    place(bi.extra(cfg->n_layers, 0), 4ull * B * H);
  }
  L.scratch_total = off;
  L.kv_layer_bytes = (uint64_t)B * Hkv * cfg->kv_capacity * hd * (cfg->kv_dtype == MK_DTYPE_F32 ? 4 : 2);

  std::vector<Op> ops = decoder_program(*cfg, bi);
  if (!bi.unfused) fuse_epilogues(ops);
  if (cfg->options & MK_LOWER_SAMPLE) {
    Op smp{OpKind::SAMPLE, bi.tokens()};
    smp.x = bi.logits();
    smp.out2 = bi.positions();
    smp.N = V;
    ops.push_back(smp);
  }

  Builder bld(L);
  std::vector<PendingTask> op;

  auto gemv = [&](const Op& o) {
    const uint16_t flags = (uint16_t)((o.gamma != kNone ? MK_FLAG_RMS_NORM_INPUT : 0) |
                                      (o.residual != kNone ? MK_FLAG_ADD_RESIDUAL : 0) | (o.silu ? MK_FLAG_SILU_MUL : 0));
    const uint32_t aux = o.gamma != kNone ? o.gamma : o.residual;
    op.clear();
    for (int64_t i = 0; i < T; ++i) {
      int64_t c0, c1;
      tile_range(o.N, T, i, mfma, c0, c1);
      PendingTask p{};
      p.d = blank();
      p.d.op_id = MK_OP_GEMV;
      p.d.config_id = (uint16_t)cfg->gemv_config;
      p.d.flags = flags;
      p.d.m = (int32_t)B;
      p.d.n = (int32_t)o.N;
      p.d.k = (int32_t)o.K;
      p.d.in_buf[0] = (uint16_t)o.x;
      p.d.in_buf[1] = (uint16_t)o.w;
      p.d.in_buf[2] = (uint16_t)aux;
      p.d.out_buf = (uint16_t)o.out;
      p.d.reserved[0] = (uint32_t)c0;
      p.d.reserved[1] = (uint32_t)(c1 - c0);
      p.d.reserved[2] = o.silu ? (uint32_t)I : 0u;
      p.reads[0] = Rect{o.x, 0, B, 0, o.K};
      p.n_reads = 1;
      if (o.residual != kNone) p.reads[p.n_reads++] = Rect{o.residual, 0, B, c0, c1};
      p.writes[0] = Rect{o.out, 0, B, c0, c1};
      p.n_writes = 1;
      op.push_back(p);
    }
    bld.emit(op);
  };

  // One task per batch row: the norm needs the whole row.
  auto norm = [&](const Op& o) {
    op.clear();
    for (int64_t b = 0; b < B; ++b) {
      PendingTask p{};
      p.d = blank();
      p.d.op_id = MK_OP_RMSNORM;
      p.d.config_id = (uint16_t)cfg->weight_dtype;
      p.d.flags = o.residual != kNone ? (uint16_t)MK_FLAG_FUSED_RESIDUAL : (uint16_t)0;
      p.d.m = (int32_t)B;
      p.d.n = (int32_t)o.N;
      p.d.in_buf[0] = (uint16_t)o.x;
      p.d.in_buf[1] = (uint16_t)o.gamma;
      p.d.in_buf[2] = (uint16_t)o.residual;
      p.d.out_buf = (uint16_t)o.out;
      p.d.reserved[0] = (uint32_t)b;
      p.d.reserved[1] = o.out2;
      p.reads[0] = Rect{o.x, b, b + 1, 0, o.N};
      p.n_reads = 1;
      p.writes[0] = Rect{o.out, b, b + 1, 0, o.N};
      p.n_writes = 1;
      if (o.residual != kNone) {
        p.reads[p.n_reads++] = Rect{o.residual, b, b + 1, 0, o.N};
        p.writes[p.n_writes++] = Rect{o.out2, b, b + 1, 0, o.N};
      }
      op.push_back(p);
    }
    bld.emit(op);
  };

  // One task per batch row after the lm_head: writes the row's greedy token and
  // advances its position.
  auto sample = [&](const Op& o) {
    op.clear();
    for (int64_t b = 0; b < B; ++b) {
      PendingTask p{};
      p.d = blank();
      p.d.op_id = MK_OP_SAMPLE;
      p.d.m = (int32_t)B;
      p.d.n = (int32_t)o.N;
      p.d.in_buf[0] = (uint16_t)o.x;
      p.d.out_buf = (uint16_t)o.out;
      p.d.reserved[0] = (uint32_t)b;
      p.d.reserved[1] = o.out2;
      p.reads[0] = Rect{o.x, b, b + 1, 0, o.N};
      p.n_reads = 1;
      p.writes[0] = Rect{o.out, b, b + 1, 0, 1};
      p.writes[1] = Rect{o.out2, b, b + 1, 0, 1};
      p.n_writes = 2;
      op.push_back(p);
    }
    bld.emit(op);
  };

  auto embed = [&](const Op& o) {
    op.clear();
    PendingTask p{};
    p.d = blank();
    p.d.op_id = MK_OP_MEMCPY;
    p.d.config_id = (uint16_t)cfg->weight_dtype;
    p.d.m = (int32_t)B;
    p.d.n = (int32_t)H;
    p.d.in_buf[0] = (uint16_t)o.x;
    p.d.in_buf[1] = (uint16_t)o.w;
    p.d.out_buf = (uint16_t)o.out;
    p.n_reads = 0;
    p.writes[0] = Rect{o.out, 0, B, 0, H};
    p.n_writes = 1;
    op.push_back(p);
    bld.emit(op);
  };

  // RoPE-append per (sequence, KV head), a partial per (sequence, KV head, chunk), a
  // combine per (sequence, KV head).
  auto attention = [&](const Op& ao) {
    const int l = ao.layer;
    const uint32_t qkv = ao.x, qrot = bi.act(l, 1), part = bi.act(l, 2), att = ao.out;
    const uint32_t kc = bi.layer(l, KCACHE), vc = bi.layer(l, VCACHE);
    op.clear();
    for (int64_t b = 0; b < B; ++b)
      for (int64_t g = 0; g < Hkv; ++g) {
        PendingTask p{};
        p.d = blank();
        p.d.op_id = MK_OP_ATTENTION_APPEND;
        p.d.config_id = kvc;
        p.d.m = (int32_t)B;
        p.d.n = (int32_t)hd;
        p.d.k = (int32_t)g;
        p.d.kv_len = cfg->kv_capacity;
        p.d.in_buf[0] = (uint16_t)qkv;
        p.d.out_buf = (uint16_t)qrot;
        p.d.reserved[0] = (uint32_t)b;
        p.d.reserved[1] = (uint32_t)(g * grp);
        p.d.reserved[2] = (uint32_t)grp;
        p.d.reserved[3] = kc;
        p.d.reserved[4] = vc;
        const int64_t q0 = g * grp * hd, k0 = Hq * hd + g * hd, v0 = (Hq + Hkv) * hd + g * hd;
        p.reads[0] = Rect{qkv, b, b + 1, q0, q0 + grp * hd};
        p.reads[1] = Rect{qkv, b, b + 1, k0, k0 + hd};
        p.reads[2] = Rect{qkv, b, b + 1, v0, v0 + hd};
        p.n_reads = 3;
        p.writes[0] = Rect{qrot, b, b + 1, q0, q0 + grp * hd};
        p.n_writes = 1;
        op.push_back(p);
      }
    bld.emit(op);

    op.clear();
    for (int64_t b = 0; b < B; ++b)
      for (int64_t g = 0; g < Hkv; ++g)
        for (int64_t c = 0; c < chunks[b]; ++c) {
          PendingTask p{};
          p.d = blank();
          p.d.op_id = MK_OP_ATTENTION_PARTIAL;
          p.d.config_id = kvc;
          p.d.m = (int32_t)chunks[b];
          p.d.n = (int32_t)hd;
          p.d.k = (int32_t)g;
          p.d.kv_len = cfg->kv_chunk;
          p.d.in_buf[0] = (uint16_t)qrot;
          p.d.in_buf[1] = (uint16_t)kc;
          p.d.in_buf[2] = (uint16_t)vc;
          p.d.out_buf = (uint16_t)part;
          const int64_t sb = slot_base[b * Hkv + g];
          p.d.reserved[0] = (uint32_t)b;
          p.d.reserved[1] = (uint32_t)(g * grp);
          p.d.reserved[2] = (uint32_t)grp;
          p.d.reserved[3] = (uint32_t)c;
          p.d.reserved[4] = (uint32_t)sb;
          const int64_t q0 = g * grp * hd;
          p.reads[0] = Rect{qrot, b, b + 1, q0, q0 + grp * hd};
          p.n_reads = 1;
          p.writes[0] = Rect{part, 0, 1, sb + c, sb + c + 1};
          p.n_writes = 1;
          op.push_back(p);
        }
    bld.emit(op);

    op.clear();
    for (int64_t b = 0; b < B; ++b)
      for (int64_t g = 0; g < Hkv; ++g) {
        PendingTask p{};
        p.d = blank();
        p.d.op_id = MK_OP_ATTENTION_COMBINE;
        p.d.m = (int32_t)chunks[b];
        p.d.n = (int32_t)hd;
        p.d.k = (int32_t)g;
        p.d.kv_len = cfg->kv_chunk;
        p.d.in_buf[0] = (uint16_t)part;
        p.d.out_buf = (uint16_t)att;
        const int64_t sb = slot_base[b * Hkv + g];
        p.d.reserved[0] = (uint32_t)b;
        p.d.reserved[1] = (uint32_t)(g * grp);
        p.d.reserved[2] = (uint32_t)grp;
        p.d.reserved[4] = (uint32_t)sb;
        const int64_t q0 = g * grp * hd;
        p.reads[0] = Rect{part, 0, 1, sb, sb + chunks[b]};
        p.n_reads = 1;
        p.writes[0] = Rect{att, b, b + 1, q0, q0 + grp * hd};
        p.n_writes = 1;
        op.push_back(p);
      }
    bld.emit(op);
  };

  for (const Op& o : ops) {
    switch (o.kind) {
      case OpKind::EMBED: embed(o); break;
      case OpKind::NORM: norm(o); break;
      case OpKind::MATMUL: gemv(o); break;
      case OpKind::ATTN: attention(o); break;
      case OpKind::SAMPLE: sample(o); break;
    }
  }
  bld.finish();
  // A NOP join never runs: its children poll its counter in place of its own
  // arrival, which only works one level deep, so a NOP must never feed another NOP.
  for (const mk_task_t& d : L.tasks)
    if (d.op_id == MK_OP_NOP)
      for (int32_t i = 0; i < d.num_dependents; ++i)
        if (L.tasks[L.edges[d.dependents_offset + i]].op_id == MK_OP_NOP)
          return set_error(MK_ERR_INVALID, "internal: a NOP join feeds another NOP join");

  BlobHeader& h = L.header;
  h.magic = 0x31474B4Du;  // "MKG1"
  h.abi_version = MK_ABI_VERSION;
  h.n_tasks = (uint32_t)L.tasks.size();
  h.n_edges = (uint32_t)L.edges.size();
  h.n_buffers = nb;
  h.rms_eps = cfg->rms_eps;
  h.rope_theta = cfg->rope_theta;
  h.kv_chunk = cfg->kv_chunk;
  h.hidden = cfg->hidden;
  h.n_q_heads = cfg->n_q_heads;
  h.n_kv_heads = cfg->n_kv_heads;
  h.head_dim = cfg->head_dim;
  h.batch = cfg->batch;
  h.intermediate = cfg->intermediate;
  h.vocab = cfg->vocab;
  h.kv_capacity = cfg->kv_capacity;
  if (L.tasks.size() >= (1u << 28)) return set_error(MK_ERR_INVALID, "graph too large (task ids need 28 bits)");
  return MK_OK;
}

// The last error message of the calling thread, in a fixed buffer: recording an
// error allocates nothing, so entry points that must not allocate can report one.
static thread_local char g_last_error[512];

int set_error(int code, const char* msg) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg ? msg : "");
  return code;
}

int set_error(int code, const std::string& msg) { return set_error(code, msg.c_str()); }

}  // namespace mk

extern "C" {

const char* mk_last_error(void) { return mk::g_last_error; }

uint32_t mk_abi_version(void) { return MK_ABI_VERSION; }

int mk_plan(const mk_model_cfg* cfg, mk_plan_info* out) {
  if (!out) return mk::set_error(MK_ERR_INVALID, "out is NULL");
  mk::Lowered L;
  int rc = mk::lower(cfg, L);
  if (rc) return rc;
  out->n_tasks = (uint32_t)L.tasks.size();
  out->n_edges = (uint32_t)L.edges.size();
  out->n_buffers = L.bi.count();
  out->n_levels = L.n_levels;
  out->scratch_bytes = L.scratch_total;
  out->kv_layer_bytes = L.kv_layer_bytes;
  return MK_OK;
}

int mk_lower(const mk_model_cfg* cfg, mk_lowered** out) {
  if (!out) return mk::set_error(MK_ERR_INVALID, "out is NULL");
  *out = nullptr;
  mk_lowered* g = new (std::nothrow) mk_lowered();
  if (!g) return mk::set_error(MK_ERR_NOMEM, "out of host memory");
  int rc;
  try {
    rc = mk::lower(cfg, g->low);
  } catch (const std::bad_alloc&) {
    rc = mk::set_error(MK_ERR_NOMEM, "out of host memory while lowering");
  }
  if (rc) {
    delete g;
    return rc;
  }
  *out = g;
  return MK_OK;
}

int mk_lowered_tasks(const mk_lowered* g, const mk_task_t** tasks, uint32_t* n) {
  if (!g || !tasks || !n) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  *tasks = g->low.tasks.data();
  *n = (uint32_t)g->low.tasks.size();
  return MK_OK;
}

int mk_lowered_edges(const mk_lowered* g, const uint32_t** edges, uint32_t* n) {
  if (!g || !edges || !n) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  *edges = g->low.edges.data();
  *n = (uint32_t)g->low.edges.size();
  return MK_OK;
}

int mk_lowered_scratch_span(const mk_lowered* g, uint32_t buf, uint64_t* offset, uint64_t* bytes) {
  if (!g || !offset || !bytes) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  if (buf >= g->low.scratch_off.size() || g->low.scratch_off[buf] == UINT64_MAX)
    return mk::set_error(MK_ERR_INVALID, "buffer is not an activation in the scratch block");
  *offset = g->low.scratch_off[buf];
  *bytes = g->low.scratch_size[buf];
  return MK_OK;
}

void mk_lowered_free(mk_lowered* g) { delete g; }

}  // extern "C"
