// C-ABI entry points of the routed MoE layer: validation, workspace layout and
// the launch sequence on the caller's stream.
#include <string.h>

#include <atomic>

#include "kernels.h"
#include "moe_mxfp4.h"

using namespace moe;

// Device scratch of moe_layer_forward_noalloc: one copy per GPU, held from the
// library's load until the process ends.  In host code `scratch` names a
// host-side stand-in, never a device address: host code uses only the
// per-device pointer that hipGetSymbolAddress returns (scratch_on_device).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// The current device's copy of `scratch`, looked up once per device (with
// that device current) and kept.  Returns a MOE_* status.
int scratch_on_device(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // concurrent first calls on one device look the address up twice and store the same value
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = (uint8_t*)p;
  return MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t z, idx, gates, counts, offsets, perm, inv, groups, n_groups, hist, done, xn, xq, xs, hq, hs, hsh, y;
  size_t xpair, xsum, hpair, hsum;  // Q2_K experts: sub-block sums of x and of h
  size_t total;
  int max_groups;  // capacity of the work list: groups of kGroupRows rows, the most there can be
};

// The shared expert runs inside the grouped GEMMs (as work-list groups) when
// it is MXFP4; a bf16 shared expert has GEMMs of its own.
bool shared_in_list(const moe_config_t& c) { return c.has_shared && c.shared_format == MOE_SHARED_MXFP4; }
bool shared_bf16(const moe_config_t& c) { return c.has_shared && c.shared_format == MOE_SHARED_BF16; }

// The bf16 shared expert streamed from its packed copy (large batches).
bool shared_stream(const moe_config_t& c, const moe_args_t& a) {
  return shared_bf16(c) && a.sh_packed && a.n_rows >= kSharedStreamRows && c.d_model % 512 == 0 &&
         c.d_ff % 256 == 0;
}

// The bf16 shared expert's GEMMs: streamed from the packed copy or tiled from sh_*_w.
hipError_t shared_gateup(const moe_config_t& c, const moe_args_t& a, const uint16_t* x, uint16_t* hsh,
                         hipStream_t stream) {
  const int N = a.n_rows, d = c.d_model, I = c.d_ff;
  if (shared_stream(c, a)) {
    const uint8_t* p = (const uint8_t*)a.sh_packed;
    return launch_shared_stream_gateup(x, N, d, I, p, p + (size_t)I * d * 2, c.swiglu_limit, hsh, stream);
  }
  return launch_shared_bf16_gateup(x, N, d, I, (const uint16_t*)a.w.sh_gate_w, (const uint16_t*)a.w.sh_up_w,
                                   c.swiglu_limit, hsh, stream);
}

hipError_t shared_down(const moe_config_t& c, const moe_args_t& a, const uint16_t* hsh, float* y_sh,
                       hipStream_t stream) {
  const int N = a.n_rows, d = c.d_model, I = c.d_ff;
  if (shared_stream(c, a))
    return launch_shared_stream_down(hsh, N, d, I, (const uint8_t*)a.sh_packed + 2 * (size_t)I * d * 2, y_sh, stream);
  return launch_shared_bf16_down(hsh, N, d, I, (const uint16_t*)a.w.sh_down_w, y_sh, stream);
}
static_assert(kSharedStreamRows == MOE_SHARED_STREAM_ROWS, "the header states the threshold");

bool q2k(const moe_config_t& c) { return c.expert_format == MOE_EXPERTS_Q2K; }

// Bytes of one routed weight matrix set [E] of [rows][K]: q and s parts.
size_t set_q_bytes(const moe_config_t& c, int rows, int K) {
  return (size_t)c.n_experts * (q2k(c) ? q2k_matrix_bytes(rows, K) : packed_q_bytes(rows, K));
}
size_t set_s_bytes(const moe_config_t& c, int rows, int K) {
  return q2k(c) ? 0 : (size_t)c.n_experts * packed_s_bytes(rows, K);
}

// Workspace carve-up; every region starts on a 256-byte boundary.
Layout make_layout(const moe_config_t& c, int n) {
  Layout L;
  const size_t N = (size_t)n, E = (size_t)c.n_experts, k = (size_t)c.top_k;
  const size_t P = N * k, Ptot = P + (c.has_shared ? N : 0), Phq = P + (shared_in_list(c) ? N : 0);
  L.max_groups = max_work_groups(n, c.top_k, c.n_experts, shared_in_list(c), kGroupRows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.z = take((size_t)logits_splits(n, c.n_experts, c.d_model) * logits_partial_stride(n, c.n_experts) * 4);
  L.idx = take(P * 4);
  L.gates = take(P * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(P * 4);
  L.inv = take(P * 4);
  L.groups = take((size_t)L.max_groups * sizeof(Group));
  L.n_groups = take(4);
  L.hist = take(route_hist_bytes(n, c.n_experts));
  L.done = take(4 * kLayerCounters);  // selection completion count, claim counters
  L.xn = take(N * (size_t)c.d_model * 2);  // the normalised input (when norm_w is given)
  const bool qk = q2k(c);
  L.xq = take(qk ? 0 : N * split_q_row_bytes(c.d_model));
  L.xs = take(qk ? 0 : N * split_s_row_bytes(c.d_model));
  L.hq = take(Phq * split_q_row_bytes(c.d_ff));  // Q2_K: h in bf16, the same bytes
  L.hs = take(qk ? 0 : Phq * split_s_row_bytes(c.d_ff));
  L.xpair = take(qk ? N * (size_t)(c.d_model / 16) * 4 : 0);
  L.xsum = take(qk ? N * (size_t)(c.d_model / 256) * 4 : 0);
  L.hpair = take(qk ? P * (size_t)(c.d_ff / 16) * 4 : 0);
  L.hsum = take(qk ? P * (size_t)(c.d_ff / 256) * 4 : 0);
  L.hsh = take(shared_bf16(c) ? N * (size_t)c.d_ff * 2 : 0);  // bf16 h of a bf16 shared expert
  L.y = take(Ptot * (size_t)c.d_model * 4);
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int check_config(const moe_config_t* c) {
  if (!c) return MOE_ERR_INVALID;
  if (c->routing != MOE_ROUTING_TOPK && c->routing != MOE_ROUTING_HASH) return MOE_ERR_INVALID;
  if (c->has_shared != 0 && c->has_shared != 1) return MOE_ERR_INVALID;
  if (c->d_model < 128 || c->d_model > 65536 || c->d_model % 128) return MOE_ERR_UNSUPPORTED;
  if (c->d_ff < 128 || c->d_ff > 65536 || c->d_ff % 128) return MOE_ERR_UNSUPPORTED;
  if (c->n_experts < 1 || c->n_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts) return MOE_ERR_UNSUPPORTED;
  if (!(c->route_scale == c->route_scale) || !(c->swiglu_limit == c->swiglu_limit)) return MOE_ERR_INVALID;
  if (!(c->norm_eps >= 0.f) || c->norm_eps == INFINITY) return MOE_ERR_INVALID;
  if (c->bias_mode != 0 && c->bias_mode != 1) return MOE_ERR_INVALID;
  if (c->shared_format != MOE_SHARED_MXFP4 && c->shared_format != MOE_SHARED_BF16) return MOE_ERR_INVALID;
  if (c->expert_format != MOE_EXPERTS_MXFP4 && c->expert_format != MOE_EXPERTS_Q2K) return MOE_ERR_INVALID;
  if (c->expert_format == MOE_EXPERTS_Q2K &&
      (c->d_model % 256 || c->d_ff % 256 || (c->has_shared && c->shared_format != MOE_SHARED_BF16)))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_mat(const void* q, const void* s) {
  if (!q || !s) return MOE_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(s, 4)) return MOE_ERR_INVALID;
  return MOE_OK;
}

// Every buffer the layer writes (out, the workspace, the optional routing
// outputs) must be disjoint from every other buffer of the call, read or
// written; the one exception is a residual that is `out` itself.  Sizes of
// the read buffers are those the layer reads: each packed weight set in full,
// the token ids and the whole tid2eid table in hash mode.
bool buffers_disjoint(const moe_config_t& c, const moe_args_t& a, const void* ws, size_t ws_bytes) {
  struct Region {
    const void* p;
    size_t n;
    bool written;
  };
  const size_t N = (size_t)a.n_rows, d = (size_t)c.d_model, I = (size_t)c.d_ff, E = (size_t)c.n_experts,
               k = (size_t)c.top_k;
  const size_t gq = packed_q_bytes(c.d_ff, c.d_model), gs = packed_s_bytes(c.d_ff, c.d_model);
  const size_t dq = packed_q_bytes(c.d_model, c.d_ff), ds = packed_s_bytes(c.d_model, c.d_ff);
  const size_t Egq = set_q_bytes(c, c.d_ff, c.d_model), Egs = set_s_bytes(c, c.d_ff, c.d_model);
  const size_t Edq = set_q_bytes(c, c.d_model, c.d_ff), Eds = set_s_bytes(c, c.d_model, c.d_ff);
  Region r[32];
  int n = 0;
  auto add = [&](const void* p, size_t bytes, bool written) {
    if (p && bytes) r[n++] = Region{p, bytes, written};
  };
  add(a.out, N * d * 2, true);
  add(ws, ws_bytes, true);
  add(a.topk_idx, N * k * 4, true);
  add(a.topk_w, N * k * 4, true);
  add(a.counts, E * 4, true);
  add(a.offsets, (E + 1) * 4, true);
  add(a.perm, N * k * 4, true);
  add(a.inv, N * k * 4, true);
  add(a.x, N * d * 2, false);
  add(a.router_w, E * d * 4, false);
  add(a.router_bias, E * 4, false);
  add(a.norm_w, a.norm_w ? d * 2 : 0, false);
  if (a.residual != a.out) add(a.residual, N * d * 2, false);
  add(a.w.gate_q, Egq, false);
  add(a.w.gate_s, Egs, false);
  add(a.w.up_q, Egq, false);
  add(a.w.up_s, Egs, false);
  add(a.w.down_q, Edq, false);
  add(a.w.down_s, Eds, false);
  if (shared_in_list(c)) {
    add(a.w.sh_gate_q, gq, false);
    add(a.w.sh_gate_s, gs, false);
    add(a.w.sh_up_q, gq, false);
    add(a.w.sh_up_s, gs, false);
    add(a.w.sh_down_q, dq, false);
    add(a.w.sh_down_s, ds, false);
  }
  if (shared_bf16(c)) {
    add(a.w.sh_gate_w, I * d * 2, false);
    add(a.w.sh_up_w, I * d * 2, false);
    add(a.w.sh_down_w, I * d * 2, false);
    add(a.sh_packed, 3 * I * d * 2, false);
  }
  if (c.routing == MOE_ROUTING_HASH) {
    add(a.token_ids, N * 4, false);
    add(a.tid2eid, (size_t)a.vocab * k * 4, false);
  }
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if ((r[i].written || r[j].written) && overlap(r[i].p, r[i].n, r[j].p, r[j].n)) return false;
  return true;
}

// Every argument check of the layer call except those on the workspace
// (host-only; nothing is enqueued).  n_rows > 0.
int check_args(const moe_config_t& c, const moe_args_t& a) {
  int rc;
  if (!a.x || !a.router_w || !a.out) return MOE_ERR_INVALID;
  if (!aligned(a.x, 16) || !aligned(a.router_w, 16) || !aligned(a.out, 16)) return MOE_ERR_INVALID;
  if (a.router_bias && !aligned(a.router_bias, 4)) return MOE_ERR_INVALID;
  if (q2k(c)) {
    const void* wq[] = {a.w.gate_q, a.w.up_q, a.w.down_q};
    for (const void* p : wq)
      if (!p || !aligned(p, 16)) return MOE_ERR_INVALID;
  } else if ((rc = check_mat(a.w.gate_q, a.w.gate_s)) || (rc = check_mat(a.w.up_q, a.w.up_s)) ||
             (rc = check_mat(a.w.down_q, a.w.down_s))) {
    return rc;
  }
  if (shared_in_list(c) && ((rc = check_mat(a.w.sh_gate_q, a.w.sh_gate_s)) ||
                             (rc = check_mat(a.w.sh_up_q, a.w.sh_up_s)) ||
                             (rc = check_mat(a.w.sh_down_q, a.w.sh_down_s))))
    return rc;
  if (shared_bf16(c)) {
    const void* shw[] = {a.w.sh_gate_w, a.w.sh_up_w, a.w.sh_down_w};
    for (const void* p : shw)
      if (!p || !aligned(p, 16)) return MOE_ERR_INVALID;
    if (a.sh_packed && !aligned(a.sh_packed, 16)) return MOE_ERR_INVALID;
  }
  if (c.routing == MOE_ROUTING_HASH) {
    if (!a.token_ids || !a.tid2eid || a.vocab < 1 || !aligned(a.token_ids, 4) || !aligned(a.tid2eid, 4))
      return MOE_ERR_INVALID;
  }
  const void* opt[] = {a.topk_idx, a.topk_w, a.counts, a.offsets, a.perm, a.inv};
  for (const void* p : opt)
    if (p && !aligned(p, 4)) return MOE_ERR_INVALID;
  if (a.norm_w && !aligned(a.norm_w, 16)) return MOE_ERR_INVALID;
  if (a.residual && !aligned(a.residual, 16)) return MOE_ERR_INVALID;
  return MOE_OK;
}

// The launch sequence with Q2_K routed experts: router logits (no activation
// split), sub-block sums of x, selection, the Q2_K gate/up GEMM writing h
// (fp16 under a swiglu clamp of at most 255, else bf16) and the bf16 shared
// expert's, sub-block sums of h, the down GEMMs and the combine.
int run_layer_q2k(const moe_config_t& c, const moe_args_t& a, uint8_t* ws, const Layout& L, hipStream_t stream) {
  const int N = a.n_rows;
  const int d = c.d_model, I = c.d_ff, E = c.n_experts, k = c.top_k;
  float* z = (float*)(ws + L.z);
  int32_t* idx = a.topk_idx ? a.topk_idx : (int32_t*)(ws + L.idx);
  float* gates = a.topk_w ? a.topk_w : (float*)(ws + L.gates);
  int32_t* counts = a.counts ? a.counts : (int32_t*)(ws + L.counts);
  int32_t* offsets = a.offsets ? a.offsets : (int32_t*)(ws + L.offsets);
  int32_t* perm = a.perm ? a.perm : (int32_t*)(ws + L.perm);
  int32_t* inv = a.inv ? a.inv : (int32_t*)(ws + L.inv);
  Group* groups = (Group*)(ws + L.groups);
  int32_t* n_groups = (int32_t*)(ws + L.n_groups);
  int32_t* hist = (int32_t*)(ws + L.hist);
  int32_t* done = (int32_t*)(ws + L.done);
  uint16_t* h = (uint16_t*)(ws + L.hq);
  uint16_t* hsh = (uint16_t*)(ws + L.hsh);
  uint32_t *xpair = (uint32_t*)(ws + L.xpair), *hpair = (uint32_t*)(ws + L.hpair);
  float *xsum = (float*)(ws + L.xsum), *hsum = (float*)(ws + L.hsum);
  float* y = (float*)(ws + L.y);
  const int P = N * k;
  auto mark = [&](int i) -> bool {
    return !a.stage_events || !a.stage_events[i] ||
           hipEventRecord((hipEvent_t)a.stage_events[i], stream) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;
  const int rows = q2k_unit_rows(P, E, d, I);
  const int max_groups = max_work_groups(N, k, E, 0, rows);
  const uint16_t* x = (const uint16_t*)a.x;
  if (a.norm_w) {
    uint16_t* xn = (uint16_t*)(ws + L.xn);
    if (launch_rmsnorm(x, (const uint16_t*)a.norm_w, N, d, c.norm_eps, xn, stream) != hipSuccess) return MOE_ERR_HIP;
    x = xn;
  }
  if (launch_prologue(x, a.router_w, N, d, E, z, nullptr, nullptr, done, false, stream) != hipSuccess ||
      launch_q2k_sums(x, N, d, false, xpair, xsum, stream) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(1)) return MOE_ERR_HIP;
  if (launch_select_route(z, a.router_bias, c.bias_mode, d, N, E, k, c.routing, a.token_ids, a.tid2eid, a.vocab, idx,
                          gates, 0, counts, offsets, perm, inv, rows, groups, n_groups, hist, done,
                          stream) != hipSuccess)
    return MOE_ERR_HIP;
  Q2kArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.w0 = (const uint8_t*)a.w.gate_q;
  ga.w1 = (const uint8_t*)a.w.up_q;
  ga.act = x;
  ga.pairs = xpair;
  ga.X = xsum;
  ga.perm = perm;
  ga.groups = groups;
  ga.n_groups = n_groups;
  ga.K = d;
  ga.R = I;
  ga.k = k;
  ga.rows = rows;
  ga.P = P;
  ga.limit = c.swiglu_limit;
  ga.h = h;
  // h in fp16 (3 more bits than bf16) when the swiglu clamp bounds it: |h| <= L^2 < 65504
  ga.h_f16 = c.swiglu_limit > 0.f && c.swiglu_limit <= 255.f;
  ga.pool = done + 1;
  if (!mark(2)) return MOE_ERR_HIP;
  if (launch_q2k_gateup(ga, max_groups, stream) != hipSuccess) return MOE_ERR_HIP;
  if (shared_bf16(c) && shared_gateup(c, a, x, hsh, stream) != hipSuccess) return MOE_ERR_HIP;
  if (!mark(3)) return MOE_ERR_HIP;
  Q2kArgs da = ga;
  da.w0 = (const uint8_t*)a.w.down_q;
  da.w1 = nullptr;
  da.act = h;
  da.pairs = hpair;
  da.X = hsum;
  da.K = I;
  da.R = d;
  da.h = nullptr;
  da.y = y;
  da.pool = done + 2;
  if (launch_q2k_sums(h, P, I, ga.h_f16 != 0, hpair, hsum, stream) != hipSuccess ||
      launch_q2k_down(da, max_groups, stream) != hipSuccess)
    return MOE_ERR_HIP;
  if (shared_bf16(c) && shared_down(c, a, hsh, y + (size_t)P * d, stream) != hipSuccess) return MOE_ERR_HIP;
  if (!mark(4)) return MOE_ERR_HIP;
  if (launch_combine(y, inv, gates, N, d, k, P, c.has_shared, c.route_scale, (const uint16_t*)a.residual,
                     (uint16_t*)a.out, stream) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(5)) return MOE_ERR_HIP;
  return MOE_OK;
}

// The launch sequence of one layer call on workspace ws (laid out as L).
int run_layer(const moe_config_t& c, const moe_args_t& a, uint8_t* ws, const Layout& L, hipStream_t stream) {
  if (q2k(c)) return run_layer_q2k(c, a, ws, L, stream);
  const int N = a.n_rows;
  const int d = c.d_model, I = c.d_ff, E = c.n_experts, k = c.top_k;
  float* z = (float*)(ws + L.z);
  int32_t* idx = a.topk_idx ? a.topk_idx : (int32_t*)(ws + L.idx);
  float* gates = a.topk_w ? a.topk_w : (float*)(ws + L.gates);
  int32_t* counts = a.counts ? a.counts : (int32_t*)(ws + L.counts);
  int32_t* offsets = a.offsets ? a.offsets : (int32_t*)(ws + L.offsets);
  int32_t* perm = a.perm ? a.perm : (int32_t*)(ws + L.perm);
  int32_t* inv = a.inv ? a.inv : (int32_t*)(ws + L.inv);
  Group* groups = (Group*)(ws + L.groups);
  int32_t* n_groups = (int32_t*)(ws + L.n_groups);
  uint8_t *xq = ws + L.xq, *xs = ws + L.xs, *hq = ws + L.hq, *hs = ws + L.hs;
  float* y = (float*)(ws + L.y);
  const int P = N * k;

  int32_t* hist = (int32_t*)(ws + L.hist);
  int32_t* done = (int32_t*)(ws + L.done);
  hipError_t err;
  auto mark = [&](int i) -> bool {
    return !a.stage_events || !a.stage_events[i] ||
           hipEventRecord((hipEvent_t)a.stage_events[i], stream) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;
  const int rows = unit_rows(P, E, d, I);
  const int max_groups = max_work_groups(N, k, E, shared_in_list(c), rows);
  const uint16_t* x = (const uint16_t*)a.x;
  if (a.norm_w) {
    uint16_t* xn = (uint16_t*)(ws + L.xn);
    if ((err = launch_rmsnorm(x, (const uint16_t*)a.norm_w, N, d, c.norm_eps, xn, stream)) != hipSuccess)
      return MOE_ERR_HIP;
    x = xn;
  }
  if ((err = launch_prologue(x, a.router_w, N, d, E, z, xq, xs, done, rows == kTallGroupRows, stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(1)) return MOE_ERR_HIP;
  if ((err = launch_select_route(z, a.router_bias, c.bias_mode, d, N, E, k, c.routing, a.token_ids, a.tid2eid, a.vocab, idx, gates, shared_in_list(c),
                                 counts, offsets, perm, inv, rows, groups, n_groups, hist, done, stream)) != hipSuccess)
    return MOE_ERR_HIP;

  ExpertArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.q0 = (const uint8_t*)a.w.gate_q;
  ga.s0 = (const uint8_t*)a.w.gate_s;
  ga.q1 = (const uint8_t*)a.w.up_q;
  ga.s1 = (const uint8_t*)a.w.up_s;
  ga.sq0 = (const uint8_t*)a.w.sh_gate_q;
  ga.ss0 = (const uint8_t*)a.w.sh_gate_s;
  ga.sq1 = (const uint8_t*)a.w.sh_up_q;
  ga.ss1 = (const uint8_t*)a.w.sh_up_s;
  ga.aq = xq;
  ga.as = xs;
  ga.perm = perm;
  ga.groups = groups;
  ga.n_groups = n_groups;
  ga.rows = rows;
  ga.K = d;
  ga.R = I;
  ga.E = E;
  ga.k = k;
  ga.P = P;
  ga.limit = c.swiglu_limit;
  ga.hq = hq;
  ga.hs = hs;
  ga.pool = done + 1;
  ga.xcd_ctr = done + 3;
  if (!mark(2)) return MOE_ERR_HIP;
  if ((err = launch_gateup(ga, max_groups, stream)) != hipSuccess) return MOE_ERR_HIP;
  uint16_t* hsh = (uint16_t*)(ws + L.hsh);
  if (shared_bf16(c) && (err = shared_gateup(c, a, x, hsh, stream)) != hipSuccess) return MOE_ERR_HIP;

  ExpertArgs da = ga;
  da.q0 = (const uint8_t*)a.w.down_q;
  da.s0 = (const uint8_t*)a.w.down_s;
  da.q1 = da.s1 = nullptr;
  da.sq0 = (const uint8_t*)a.w.sh_down_q;
  da.ss0 = (const uint8_t*)a.w.sh_down_s;
  da.sq1 = da.ss1 = nullptr;
  da.aq = hq;
  da.pool = done + 2;
  da.xcd_ctr = done + 3 + kXcds;
  da.as = hs;
  da.K = I;
  da.R = d;
  da.hq = da.hs = nullptr;
  da.y = y;
  if (!mark(3)) return MOE_ERR_HIP;
  if ((err = launch_down(da, max_groups, stream)) != hipSuccess) return MOE_ERR_HIP;
  if (shared_bf16(c) && (err = shared_down(c, a, hsh, y + (size_t)P * d, stream)) != hipSuccess) return MOE_ERR_HIP;
  if (!mark(4)) return MOE_ERR_HIP;

  if ((err = launch_combine(y, inv, gates, N, d, k, P, c.has_shared, c.route_scale, (const uint16_t*)a.residual,
                            (uint16_t*)a.out, stream)) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(5)) return MOE_ERR_HIP;
  return MOE_OK;
}


}  // namespace

extern "C" {

int moe_version(void) { return MOE_MXFP4_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "call needs more than the library's static scratch (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int moe_packed_mxfp4_bytes(int32_t rows, int32_t K, size_t* q_bytes, size_t* s_bytes) {
  if (!q_bytes || !s_bytes) return MOE_ERR_INVALID;
  if (rows < 16 || rows % 16 || K < 128 || K % 128) return MOE_ERR_UNSUPPORTED;
  *q_bytes = packed_q_bytes(rows, K);
  *s_bytes = packed_s_bytes(rows, K);
  return MOE_OK;
}

int moe_pack_mxfp4(const void* q, const void* s, int32_t n_mat, int32_t rows, int32_t K, void* q_out, void* s_out,
                   void* stream) {
  if (n_mat < 0) return MOE_ERR_INVALID;
  if (rows < 16 || rows % 16 || K < 128 || K % 128 || rows > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  if (n_mat == 0) return MOE_OK;
  if (!q || !s || !q_out || !s_out) return MOE_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(s_out, 4)) return MOE_ERR_INVALID;
  const size_t nq = (size_t)n_mat * packed_q_bytes(rows, K);
  const size_t ns_in = (size_t)n_mat * rows * (K / 32), ns_out = (size_t)n_mat * packed_s_bytes(rows, K);
  if (overlap(q, nq, q_out, nq) || overlap(s, ns_in, s_out, ns_out) || overlap(q, nq, s_out, ns_out) ||
      overlap(s, ns_in, q_out, nq))
    return MOE_ERR_INVALID;
  hipError_t err = launch_pack_mxfp4((const uint8_t*)q, (const uint8_t*)s, n_mat, rows, K, (uint8_t*)q_out,
                                     (uint8_t*)s_out, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_pack_bf16(const void* w, int32_t n_mat, int32_t rows, int32_t K, void* out, void* stream) {
  if (n_mat < 0) return MOE_ERR_INVALID;
  if (rows < 16 || rows % 16 || K < 32 || K % 32 || rows > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  if (n_mat == 0) return MOE_OK;
  if (!w || !out || !aligned(w, 16) || !aligned(out, 16)) return MOE_ERR_INVALID;
  const size_t n = (size_t)n_mat * rows * K * 2;
  if (overlap(w, n, out, n)) return MOE_ERR_INVALID;
  hipError_t err = launch_pack_bf16((const uint8_t*)w, n_mat, rows, K, (uint8_t*)out, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_q2k_bytes(int32_t rows, int32_t K, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID;
  if (rows < 16 || rows % 16 || K < 256 || K % 256) return MOE_ERR_UNSUPPORTED;
  *bytes = q2k_matrix_bytes(rows, K);
  return MOE_OK;
}

int moe_pack_q2k(const void* q, int32_t n_mat, int32_t rows, int32_t K, void* q_out, void* stream) {
  if (n_mat < 0) return MOE_ERR_INVALID;
  if (rows < 16 || rows % 16 || K < 256 || K % 256 || rows > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  if (n_mat == 0) return MOE_OK;
  if (!q || !q_out || !aligned(q, 4) || !aligned(q_out, 16)) return MOE_ERR_INVALID;
  const size_t n = (size_t)n_mat * q2k_matrix_bytes(rows, K);
  if (overlap(q, n, q_out, n)) return MOE_ERR_INVALID;
  return launch_pack_q2k((const uint8_t*)q, n_mat, rows, K, (uint8_t*)q_out, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

int moe_workspace_size(const moe_config_t* cfg, int32_t n_rows, size_t* bytes) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!bytes || n_rows < 0) return MOE_ERR_INVALID;
  if (n_rows > MOE_MAX_ROWS) return MOE_ERR_UNSUPPORTED;
  *bytes = n_rows == 0 ? 0 : make_layout(*cfg, n_rows).total;
  return MOE_OK;
}

int moe_layer_forward(const moe_config_t* cfg, const moe_args_t* args, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!args) return MOE_ERR_INVALID;
  const moe_config_t& c = *cfg;
  const moe_args_t& a = *args;
  if (a.n_rows < 0) return MOE_ERR_INVALID;
  if (a.n_rows > MOE_MAX_ROWS) return MOE_ERR_UNSUPPORTED;
  if (a.n_rows == 0) return MOE_OK;
  if ((rc = check_args(c, a))) return rc;
  const Layout L = make_layout(c, a.n_rows);
  if (!a.workspace || a.workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(a.workspace, 256)) return MOE_ERR_INVALID;
  if (!buffers_disjoint(c, a, a.workspace, L.total)) return MOE_ERR_INVALID;
  return run_layer(c, a, (uint8_t*)a.workspace, L, (hipStream_t)stream);
}

int moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_args_t* args, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!args) return MOE_ERR_INVALID;
  const moe_config_t& c = *cfg;
  const moe_args_t& a = *args;
  if (a.n_rows < 0) return MOE_ERR_INVALID;
  if (a.n_rows > MOE_MAX_ROWS) return MOE_ERR_UNSUPPORTED;
  if (a.workspace || a.workspace_bytes) return MOE_ERR_INVALID;  // the library's scratch replaces it
  if (a.n_rows == 0) return MOE_OK;
  if ((rc = check_args(c, a))) return rc;
  const Layout L = make_layout(c, a.n_rows);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  // the scratch is a separate allocation of the library, so only the caller's buffers can overlap
  if (!buffers_disjoint(c, a, nullptr, 0)) return MOE_ERR_INVALID;
  uint8_t* ws = nullptr;
  if ((rc = scratch_on_device(&ws))) return rc;
  return run_layer(c, a, ws, L, (hipStream_t)stream);
}

}  // extern "C"
