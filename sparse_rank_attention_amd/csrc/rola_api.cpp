// rola_api.cpp -- host side of librola: argument validation, workspace
// planning and kernel launch sequences for the four entry points of rola.h.
//
// Every entry point validates all of its arguments before it launches
// anything, so a call either launches nothing (status != ROLA_OK) or
// enqueues its whole kernel sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rola.h"
#include "rola_internal.h"

namespace {

constexpr int64_t kAlign = 256;
constexpr int kBlkParts = 32;  // complement scope: block-range partials of the global state

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ plan
struct Plan {
  int B, H, D, r, kb, nb;
  int64_t N, n_pad, BH;
  int split[3];
  double theta;
  float scale;
  int grid[3];
  int nchunks, cpc;
  // workspace offsets (bytes)
  int G;
  int64_t ngroups, list_stride;
  int64_t off_wqT, off_wkT, off_qp, off_kp, off_scores, off_map, off_part, off_st,
      off_z, off_ugroup, off_ucount, off_ulist, total;
  bool fp8;
  int64_t off_qsc, off_ksc, off_vsc, off_kv8;  // fp8 only
  bool vh;  // bf16 output, bf16 operands: the fp16 copy of V and its range flags
  int64_t off_vh, off_vovf;
  bool comp;  // complement scope of the low-rank branch
  int64_t off_blk, off_s32, off_stc, off_zc;  // complement scope only
  // rola_backward: its buffers follow the forward's (offsets from 0)
  int64_t b_os, b_os_elems, b_lse, b_dob, b_dn, b_dqp, b_dkp, b_dvp, b_ahat, b_duq, b_dwk, b_dy, b_dg,
      b_wqP, b_wkP, b_sd, b_dsr, b_dst, b_ds32, b_dz, b_s32, b_part, b_tcount, b_tlist, b_tbits, b_sumtmp, total_bwd;
  int64_t b_sdc, b_pblk, b_dzblk, b_dsrc, b_dstc, b_dzc;  // complement scope only
};

int32_t make_plan(const rola_problem *p, const rola_config *c, Plan *pl) {
  if (!p || !c || !pl) return ROLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads < 1 || p->grid_t < 1 || p->grid_h < 1 || p->grid_w < 1)
    return ROLA_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return ROLA_ERR_UNSUPPORTED;
  if (c->rank != 16 && c->rank != 32) return ROLA_ERR_UNSUPPORTED;
  if (c->precision != ROLA_PREC_BF16 && c->precision != ROLA_PREC_FP8) return ROLA_ERR_INVALID_ARG;
  if (c->out_dtype != ROLA_OUT_BF16 && c->out_dtype != ROLA_OUT_F32) return ROLA_ERR_INVALID_ARG;
  if (c->lowrank_scope != ROLA_LR_GLOBAL && c->lowrank_scope != ROLA_LR_COMPLEMENT)
    return ROLA_ERR_INVALID_ARG;
  const int D = p->head_dim;
  const int64_t N = (int64_t)p->grid_t * p->grid_h * p->grid_w;
  const int64_t nb64 = (N + ROLA_BLOCK - 1) / ROLA_BLOCK;
  if (nb64 > ROLA_MAX_BLOCKS) return ROLA_ERR_UNSUPPORTED;
  const int nb = (int)nb64;
  // strides: 16-byte aligned rows, rows at least D long
  if (p->stride_n < D || p->stride_n % 8 || p->stride_h % 8 || p->stride_b % 8 ||
      p->stride_h < 0 || p->stride_b < 0)
    return ROLA_ERR_ALIGNMENT;
  // byte offsets inside one 64-token block are 32-bit in the tile copies
  if (p->stride_n > (1LL << 24)) return ROLA_ERR_UNSUPPORTED;
  int kb;
  if (c->kb_override > 0) {
    if (c->kb_override > nb) return ROLA_ERR_INVALID_ARG;
    kb = c->kb_override;
  } else {
    if (!(c->topk > 0.0f && c->topk <= 1.0f)) return ROLA_ERR_INVALID_ARG;
    // floor(topk * nb) with a relative allowance of 2^-22 for the float32
    // rounding of a decimal keep ratio (at most 2^-24 of it)
    const double prod = (double)c->topk * nb;
    const double kk = std::floor(prod + std::ldexp(prod, -22));
    kb = (int)std::max(1.0, std::min((double)nb, kk));
  }
  if (c->kb_override < 0) return ROLA_ERR_INVALID_ARG;
  int split[3] = {c->rope_split[0], c->rope_split[1], c->rope_split[2]};
  if (split[0] == 0 && split[1] == 0 && split[2] == 0) {
    split[0] = D / 4;
    split[1] = (D - split[0]) / 2;
    split[2] = D - split[0] - split[1];
  }
  for (int a = 0; a < 3; ++a)
    if (split[a] < 0 || split[a] % 2) return ROLA_ERR_INVALID_ARG;
  if (split[0] + split[1] + split[2] != D) return ROLA_ERR_INVALID_ARG;
  if (std::isnan(c->rope_theta) || std::isnan(c->softmax_scale) || std::isinf(c->softmax_scale) ||
      std::isinf(c->rope_theta))
    return ROLA_ERR_INVALID_ARG;

  Plan &P = *pl;
  P.B = p->batch; P.H = p->heads; P.D = D; P.r = c->rank; P.kb = kb; P.nb = nb;
  P.N = N; P.n_pad = (int64_t)nb * ROLA_BLOCK; P.BH = (int64_t)P.B * P.H;
  for (int a = 0; a < 3; ++a) P.split[a] = split[a];
  P.theta = c->rope_theta > 0.0f ? (double)c->rope_theta : 10000.0;
  P.scale = c->softmax_scale > 0.0f ? c->softmax_scale : (float)(1.0 / std::sqrt((double)D));
  P.grid[0] = p->grid_t; P.grid[1] = p->grid_h; P.grid[2] = p->grid_w;
  // pass-1 chunking: about 4096 workgroups in total
  int nchunks = (int)std::max<int64_t>(1, std::min<int64_t>(nb, (4096 + P.BH - 1) / P.BH));
  P.cpc = (nb + nchunks - 1) / nchunks;
  P.nchunks = (nb + P.cpc - 1) / P.cpc;

  int64_t o = 0;
  P.off_wqT = o; o = align_up(o + 32LL * D * 2);
  P.off_wkT = o; o = align_up(o + 32LL * D * 2);
  P.off_qp = o; o = align_up(o + P.BH * nb * D * 4);
  P.off_kp = o; o = align_up(o + P.BH * nb * D * 4);
  P.off_scores = o; o = align_up(o + P.BH * nb * (int64_t)nb * 4);
  P.off_map = o; o = align_up(o + P.BH * nb * (int64_t)kb * 4);
  // state partials: 2 per chunk, or (complement scope) up to kBlkParts block-range sums
  P.comp = c->lowrank_scope == ROLA_LR_COMPLEMENT;
  const int64_t nparts = std::max<int64_t>(2LL * P.nchunks, P.comp ? std::min(nb, kBlkParts) : 0);
  P.off_part = o; o = align_up(o + P.BH * nparts * (int64_t)(D * 32 + 32) * 4);
  P.off_st = o; o = align_up(o + P.BH * D * 32LL * 2);
  P.off_z = o; o = align_up(o + P.BH * 32LL * 4);
  P.G = rola::attn_group_size();
  P.ngroups = (nb + P.G - 1) / P.G;
  P.list_stride = (int64_t)P.G * kb;
  P.off_ugroup = o; o = align_up(o + P.BH * P.ngroups * P.G * 4);
  P.off_ucount = o; o = align_up(o + P.BH * P.ngroups * 4);
  P.off_ulist = o; o = align_up(o + P.BH * P.ngroups * P.list_stride * 4);
  P.fp8 = c->precision == ROLA_PREC_FP8;
  P.off_qsc = P.off_ksc = P.off_vsc = P.off_kv8 = 0;
  if (P.fp8) {
    P.off_qsc = o; o = align_up(o + P.BH * nb * 8);
    P.off_ksc = o; o = align_up(o + P.BH * nb * 4);
    P.off_vsc = o; o = align_up(o + P.BH * nb * 4);
    P.off_kv8 = o; o = align_up(o + P.BH * nb * 64LL * D);
  }
  P.vh = !P.fp8 && c->out_dtype == ROLA_OUT_BF16;
  P.off_vh = P.off_vovf = 0;
  if (P.fp8) {  // the V codes as fp16 values
    P.off_vh = o; o = align_up(o + P.BH * P.n_pad * D * 2);
  }
  if (P.vh) {
    P.off_vh = o; o = align_up(o + P.BH * P.n_pad * D * 2);
    P.off_vovf = o; o = align_up(o + P.BH * 2 * P.nchunks * 4);
  }
  P.off_blk = P.off_s32 = P.off_stc = P.off_zc = 0;
  if (P.comp) {
    P.off_blk = o; o = align_up(o + P.BH * nb * (int64_t)(D * 64 + 128));  // bf16 S^T, fp32 z
    P.off_s32 = o; o = align_up(o + P.BH * D * 32LL * 4);
    P.off_stc = o; o = align_up(o + P.BH * nb * (int64_t)D * 32 * 2);
    P.off_zc = o; o = align_up(o + P.BH * nb * 32LL * 4);
  }
  P.total = o;

  // backward buffers
  const int64_t tok = P.BH * P.n_pad;
  // the recomputed sparse output uses the problem's strides (the attention
  // kernel writes O through them): its extent in elements
  P.b_os_elems = (int64_t)(P.B - 1) * p->stride_b + (int64_t)(P.H - 1) * p->stride_h +
                 (P.n_pad - 1) * p->stride_n + D;
  const int64_t pp = rola::bwd_outer_parts(P.BH, nb, 0);
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  P.b_os = take(P.b_os_elems * 4);
  P.b_lse = take(tok * 4);
  P.b_dob = take(tok * D * 2);
  P.b_dn = take(tok * 4);
  P.b_dqp = take(tok * D * 4);
  P.b_dkp = take(tok * D * 4);
  P.b_dvp = take(tok * D * 4);
  P.b_ahat = take(tok * 32 * 2);
  P.b_duq = take(tok * 32 * 2);
  P.b_dwk = take(tok * 32 * 2);
  P.b_dy = take(tok * 4);
  P.b_dg = take(tok * 4);
  P.b_wqP = take(D * 32 * 2);
  P.b_wkP = take(D * 32 * 2);
  P.b_sd = take(P.BH * 32 * D * 2 * 2);  // hi, then lo
  P.b_dsr = take(P.BH * 32 * D * 2);
  P.b_dst = take(P.BH * D * 32 * 2);
  P.b_ds32 = take(P.BH * D * 32 * 4);
  P.b_dz = take(P.BH * 32 * 4);
  P.b_s32 = take(P.BH * D * 32 * 4);
  P.b_part = take((P.BH * pp * 4 * (int64_t)D * 32 + P.BH) * 4);
  P.b_tcount = take(P.BH * nb * 4);
  P.b_tlist = take(P.BH * nb * (int64_t)nb * 4);
  P.b_tbits = take(P.BH * nb * (int64_t)((nb + 31) / 32) * 4);
  P.b_sumtmp = take(P.BH * D * 32LL * 4);
  P.b_sdc = P.b_pblk = P.b_dzblk = P.b_dsrc = P.b_dstc = P.b_dzc = 0;
  if (P.comp) {
    const int64_t blocks = P.BH * nb;
    P.b_sdc = take(blocks * 32 * D * 2 * 2);  // hi, then lo
    P.b_pblk = take(blocks * D * 32 * 2);
    P.b_dzblk = take(blocks * 32 * 4);
    P.b_dsrc = take(blocks * 32 * D * 2);
    P.b_dstc = take(blocks * D * 32 * 2);
    P.b_dzc = take(blocks * 32 * 4);
  }
  P.total_bwd = o;
  return ROLA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------- timing
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};
// The only process-wide state of the library: the measurement aid below.
// While it is off (the default), a call reads this one flag and nothing else.
std::mutex g_mu;
std::atomic<bool> g_timing{false};
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_free_events;
constexpr size_t kEventPool = 512;  // enough for about 36 timed forward calls

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` on stream `st`, bracketed by events when timing is on.
template <typename F>
int32_t timed(const char *name, hipStream_t st, F &&launch) {
  hipEvent_t a = nullptr, b = nullptr;
  const bool on = g_timing.load(std::memory_order_relaxed);
  if (on) {
    std::lock_guard<std::mutex> lk(g_mu);
    a = take_event();
    b = take_event();
    if (a) (void)hipEventRecord(a, st);
  }
  launch();
  hipError_t err = hipGetLastError();
  if (on && a && b) {
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_mu);
    g_launches.push_back({name, a, b});
  }
  return err == hipSuccess ? ROLA_OK : ROLA_ERR_DEVICE;
}

rola::RopeArgsHost rope_args(const Plan &P, uint8_t *) {
  rola::RopeArgsHost r;
  r.off1 = P.split[0];
  r.off2 = P.split[0] + P.split[1];
  r.half0 = P.split[0] / 2;
  r.half1 = P.split[1] / 2;
  r.half2 = P.split[2] / 2;
  r.grid_h = P.grid[1];
  r.grid_w = P.grid[2];
  r.log2_theta = (float)std::log2(P.theta);
  return r;
}

int32_t run_setup(const Plan &P, const float *wq, const float *wk, uint8_t *ws, hipStream_t st) {
  rola::SetupArgs a;
  a.wq = wq; a.wk = wk; a.D = P.D; a.rank = P.r;
  a.wqT = (uint16_t *)(ws + P.off_wqT);
  a.wkT = (uint16_t *)(ws + P.off_wkT);
  return timed("setup", st, [&] { rola::launch_setup(a, st); });
}

// vh: also the fp16 copy of V with its range flags (bf16 output); with
// neither pool nor state, the copy alone
int32_t run_pass1(const Plan &P, const rola_problem *p, const void *q, const void *k, const void *v,
                  uint8_t *ws, bool pool, bool state, hipStream_t st, bool quant = false, bool vh = false) {
  rola::Pass1Args a;
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k; a.v = (const uint16_t *)v;
  a.stride_b = p->stride_b; a.stride_h = p->stride_h; a.stride_n = p->stride_n;
  a.heads = P.H; a.nb = P.nb; a.n_tokens = P.N; a.cpc = P.cpc; a.rank = P.r;
  const int64_t tail = P.N - (int64_t)(P.nb - 1) * ROLA_BLOCK;
  a.inv_tail = 1.0f / (float)tail;
  a.qp = (float *)(ws + P.off_qp);
  a.kp = (float *)(ws + P.off_kp);
  a.wkT = (const uint16_t *)(ws + P.off_wkT);
  a.state_part = (float *)(ws + P.off_part);
  a.blk_state = (P.comp && pool && state) ? ws + P.off_blk : nullptr;
  a.rope = rope_args(P, ws);
  a.qsc = (float *)(ws + P.off_qsc);
  a.ksc = (float *)(ws + P.off_ksc);
  a.vsc = (float *)(ws + P.off_vsc);
  a.kv8 = ws + P.off_kv8;
  a.vh = (vh || (quant && P.fp8)) ? (uint16_t *)(ws + P.off_vh) : nullptr;
  a.vovf = vh ? (int32_t *)(ws + P.off_vovf) : nullptr;
  if (!pool && !state)
    return timed("v_fp16", st, [&] { rola::launch_pass1(a, P.D, P.nchunks, (int)P.BH, false, false, false, st); });
  const char *name = (pool && state) ? (quant ? (a.blk_state ? "pass1_pool_blkstate_quant8"
                                                            : "pass1_pool_state_quant8")
                                              : (a.blk_state ? "pass1_pool_blkstate" : "pass1_pool_state"))
                     : pool          ? "pass1_pool"
                                     : "pass1_state";
  return timed(name, st, [&] { rola::launch_pass1(a, P.D, P.nchunks, (int)P.BH, pool, state, quant, st); });
}

int32_t run_reduce(const Plan &P, uint8_t *ws, hipStream_t st) {
  int np = 2 * P.nchunks;
  if (P.comp) {
    // pass 1 wrote per-block states instead of chunk partials: sum them over
    // block ranges first (into the chunk-partial space, which holds at least
    // min(nb, kBlkParts) partials per head)
    np = std::min<int>(P.nb, kBlkParts);
    int32_t s = timed("blk_partial", st, [&] {
      rola::launch_blk_partial(ws + P.off_blk, P.nb, np, P.D, (int)P.BH, (float *)(ws + P.off_part), st);
    });
    if (s != ROLA_OK) return s;
  }
  return timed("state_reduce", st, [&] {
    rola::launch_state_reduce((const float *)(ws + P.off_part), np, P.D, P.r, (int)P.BH,
                              (uint16_t *)(ws + P.off_st), (float *)(ws + P.off_z),
                              P.comp ? (float *)(ws + P.off_s32) : nullptr, st);
  });
}

int32_t run_select(const Plan &P, uint8_t *ws, float *scores, int32_t *map, hipStream_t st) {
  int32_t s = timed("scores", st, [&] {
    rola::launch_scores((const float *)(ws + P.off_qp), (const float *)(ws + P.off_kp), scores, P.nb,
                        P.D, (int)P.BH, st);
  });
  if (s != ROLA_OK) return s;
  return timed("topk", st, [&] { rola::launch_topk(scores, map, P.nb, P.kb, P.BH * P.nb, st); });
}

// fp8 operands of the sparse branch: quantised from bf16 q, k, v, or (when
// k8 is set) the caller's codes q8, k8, v8 and scales qs, ks, vs laid out
int32_t run_quant8(const Plan &P, const rola_problem *p, const void *q, const void *k, const void *v,
                   uint8_t *ws, hipStream_t st, const uint8_t *q8 = nullptr, const uint8_t *k8 = nullptr,
                   const uint8_t *v8 = nullptr, const float *qs = nullptr, const float *ks = nullptr,
                   const float *vs = nullptr) {
  rola::Quant8Args a;
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k; a.v = (const uint16_t *)v;
  a.q8 = q8; a.k8 = k8; a.v8 = v8;
  a.qs_in = qs; a.ks_in = ks; a.vs_in = vs;
  a.stride_b = p->stride_b; a.stride_h = p->stride_h; a.stride_n = p->stride_n;
  a.heads = P.H; a.nb = P.nb; a.n_tokens = P.N;
  a.qsc = (float *)(ws + P.off_qsc);
  a.ksc = (float *)(ws + P.off_ksc);
  a.vsc = (float *)(ws + P.off_vsc);
  a.kv8 = ws + P.off_kv8;
  a.vh = (uint16_t *)(ws + P.off_vh);
  return timed(k8 ? "image8" : "quant8", st, [&] { rola::launch_quant8(a, P.D, (int)P.BH, st); });
}

// the group schedule of a block map alone (what run_attn forms first)
int32_t run_schedule(const Plan &P, const int32_t *map, uint8_t *ws, hipStream_t st) {
  return timed("schedule", st, [&] {
    rola::launch_schedule(map, P.nb, P.kb, P.G, (int)P.ngroups, (int)P.list_stride, (int)P.BH,
                          (int32_t *)(ws + P.off_ugroup), (int32_t *)(ws + P.off_ucount),
                          (int32_t *)(ws + P.off_ulist), st);
  });
}

int32_t run_attn(const Plan &P, const rola_problem *p, const rola_config *c, const void *q,
                 const void *k, const void *v, const int32_t *map, const float *gate, void *out,
                 uint8_t *ws, bool sparse, bool lowrank, bool accum, hipStream_t st,
                 float *lse = nullptr, const uint8_t *q8 = nullptr, float *os_save = nullptr) {
  rola::AttnArgs a;
  a.q8 = q8;
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k; a.v = (const uint16_t *)v;
  a.out = out;
  a.stride_b = p->stride_b; a.stride_h = p->stride_h; a.stride_n = p->stride_n;
  a.heads = P.H; a.nb = P.nb; a.kb = P.kb; a.rank = P.r; a.n_tokens = P.N;
  a.bh_count = P.BH;
  a.ngroups = P.ngroups;
  a.groups_per_xcd = (P.ngroups + 7) / 8;
  a.list_stride = P.list_stride;
  a.ugroup = (const int32_t *)(ws + P.off_ugroup);
  a.ucount = (const int32_t *)(ws + P.off_ucount);
  a.ulist = (const int32_t *)(ws + P.off_ulist);
  a.scale_log2e = (float)((double)P.scale * 1.4426950408889634);
  a.wqT = (const uint16_t *)(ws + P.off_wqT);
  a.st = (const uint16_t *)(ws + P.off_st);
  a.z = (const float *)(ws + P.off_z);
  a.gate = lowrank ? gate : nullptr;
  a.complement = (lowrank && P.comp) ? 1 : 0;
  // bf16 output of the sparse branch: PV on the fp16 copy of V (written by
  // pass 1 or the copy pass beforehand), the EXACT form for flagged heads
  const bool f16v = sparse && !P.fp8 && c->out_dtype == ROLA_OUT_BF16;
  if (f16v && !P.vh) return ROLA_ERR_INVALID_ARG;  // (the plan of the same config holds the copy)
  a.vh = (f16v || (sparse && P.fp8)) ? (const uint16_t *)(ws + P.off_vh) : nullptr;
  a.vovf = f16v ? (const int32_t *)(ws + P.off_vovf) : nullptr;
  a.nflags = 2 * P.nchunks;
  // the log-sum-exp: the backward's recompute (sparse alone) or a training
  // forward (fused, which also keeps O_s)
  a.lse = sparse ? lse : nullptr;
  a.os_save = (sparse && lowrank) ? os_save : nullptr;
  a.rope = rope_args(P, ws);
  a.kv8 = ws + P.off_kv8;
  a.qsc = (const float *)(ws + P.off_qsc);
  a.ksc = (const float *)(ws + P.off_ksc);
  a.vsc = (const float *)(ws + P.off_vsc);
  if (sparse || a.complement) {
    int32_t s = timed("schedule", st, [&] {
      rola::launch_schedule(map, P.nb, P.kb, P.G, (int)P.ngroups, (int)P.list_stride, (int)P.BH,
                            (int32_t *)(ws + P.off_ugroup), (int32_t *)(ws + P.off_ucount),
                            (int32_t *)(ws + P.off_ulist), st);
    });
    if (s != ROLA_OK) return s;
  } else {
    // low-rank only: each "group" is one query block per member slot, in order
    int32_t s = timed("schedule", st, [&] {
      rola::launch_schedule(nullptr, P.nb, 0, P.G, (int)P.ngroups, 0, (int)P.BH,
                            (int32_t *)(ws + P.off_ugroup), (int32_t *)(ws + P.off_ucount),
                            (int32_t *)(ws + P.off_ulist), st);
    });
    if (s != ROLA_OK) return s;
  }
  if (a.complement) {
    // per query block: the global state minus the states of its kept blocks
    rola::CompArgs ca;
    ca.blk = ws + P.off_blk;
    ca.s32 = (const float *)(ws + P.off_s32);
    ca.z = (const float *)(ws + P.off_z);
    ca.ugroup = a.ugroup; ca.ucount = a.ucount; ca.ulist = a.ulist;
    ca.nb = P.nb; ca.kb = P.kb;
    ca.bh_count = P.BH; ca.ngroups = P.ngroups; ca.groups_per_xcd = a.groups_per_xcd;
    ca.list_stride = P.list_stride;
    ca.stc = (uint16_t *)(ws + P.off_stc);
    ca.zc = (float *)(ws + P.off_zc);
    ca.sdc = nullptr;
    int32_t s = timed("complement", st, [&] { rola::launch_complement(ca, P.D, st); });
    if (s != ROLA_OK) return s;
    a.st = ca.stc;
    a.z = ca.zc;
  }
  if (sparse && P.fp8) {
    const char *name8 = lowrank ? "attn8_sparse_lowrank" : "attn8_sparse";
    return timed(name8, st, [&] {
      rola::launch_attn8(a, P.D, lowrank, accum != 0, c->out_dtype == ROLA_OUT_F32, st);
    });
  }
  const char *name = sparse && lowrank ? "attn_sparse_lowrank" : sparse ? "attn_sparse" : "attn_lowrank";
  return timed(name, st, [&] {
    rola::launch_attn(a, P.D, sparse, lowrank, accum != 0, c->out_dtype == ROLA_OUT_F32, st);
  });
}

#define ROLA_TRY(x)                  \
  do {                               \
    int32_t _s = (x);                \
    if (_s != ROLA_OK) return _s;    \
  } while (0)

}  // namespace

// ---------------------------------------------------------------- C ABI
extern "C" {

int32_t rola_abi_version(void) { return ROLA_ABI_VERSION; }

const char *rola_status_str(int32_t s) {
  switch (s) {
    case ROLA_OK: return "ok";
    case ROLA_ERR_INVALID_ARG: return "invalid argument";
    case ROLA_ERR_UNSUPPORTED: return "unsupported problem (head_dim, rank, precision or size)";
    case ROLA_ERR_ALIGNMENT: return "pointer or stride not 16-byte aligned";
    case ROLA_ERR_WORKSPACE: return "workspace missing or too small";
    case ROLA_ERR_DEVICE: return "HIP launch error";
    default: return "unknown status";
  }
}

int32_t rola_plan(const rola_problem *prob, const rola_config *cfg, rola_plan_info *out) {
  if (!out) return ROLA_ERR_INVALID_ARG;
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  out->n_tokens = P.N;
  out->nb = P.nb;
  out->kb = P.kb;
  out->n_pad = P.n_pad;
  out->workspace_bytes = P.total;
  out->workspace_bytes_backward = P.total_bwd;
  return ROLA_OK;
}

int32_t rola_select_blocks(const rola_problem *prob, const rola_config *cfg, const void *q,
                           const void *k, int32_t *block_idx, float *pooled_scores,
                           void *workspace, size_t workspace_bytes, void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (!q || !k || !block_idx) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(block_idx) ||
      (pooled_scores && !aligned16(pooled_scores)))
    return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  ROLA_TRY(run_pass1(P, prob, q, k, nullptr, ws, true, false, st));
  float *scores = pooled_scores ? pooled_scores : (float *)(ws + P.off_scores);
  return run_select(P, ws, scores, block_idx, st);
}

int32_t rola_sparse_attn(const rola_problem *prob, const rola_config *cfg, const void *q,
                         const void *k, const void *v, const int32_t *block_idx, void *out,
                         int32_t accumulate, void *workspace, size_t workspace_bytes,
                         void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (!q || !k || !v || !block_idx || !out) return ROLA_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(block_idx))
    return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  if (P.fp8) ROLA_TRY(run_quant8(P, prob, q, k, v, ws, st));
  if (P.vh) ROLA_TRY(run_pass1(P, prob, nullptr, nullptr, v, ws, false, false, st, false, true));
  return run_attn(P, prob, cfg, q, k, v, block_idx, nullptr, out, ws, true, false, accumulate != 0,
                  st);
}

int32_t rola_lowrank_attn(const rola_problem *prob, const rola_config *cfg, const void *q,
                          const void *k, const void *v, const float *wq, const float *wk,
                          const float *gate, void *out, int32_t accumulate, void *workspace,
                          size_t workspace_bytes, void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (!q || !k || !v || !wq || !wk || !out) return ROLA_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ROLA_ERR_ALIGNMENT;
  if (((uintptr_t)wq & 3u) || ((uintptr_t)wk & 3u)) return ROLA_ERR_ALIGNMENT;
  if (gate && !aligned16(gate)) return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  ROLA_TRY(run_setup(P, wq, wk, ws, st));
  if (P.comp) {
    // the complement needs the block map: pool Q and K in the same pass
    ROLA_TRY(run_pass1(P, prob, q, k, v, ws, true, true, st));
    ROLA_TRY(run_reduce(P, ws, st));
    int32_t *map = (int32_t *)(ws + P.off_map);
    ROLA_TRY(run_select(P, ws, (float *)(ws + P.off_scores), map, st));
    return run_attn(P, prob, cfg, q, nullptr, nullptr, map, gate, out, ws, false, true,
                    accumulate != 0, st);
  }
  ROLA_TRY(run_pass1(P, prob, nullptr, k, v, ws, false, true, st));
  ROLA_TRY(run_reduce(P, ws, st));
  return run_attn(P, prob, cfg, q, nullptr, nullptr, nullptr, gate, out, ws, false, true,
                  accumulate != 0, st);
}

int32_t rola_forward(const rola_problem *prob, const rola_config *cfg, const void *q,
                     const void *k, const void *v, const float *wq, const float *wk,
                     const float *gate, int32_t *block_idx_out, void *out, void *workspace,
                     size_t workspace_bytes, void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (!q || !k || !v || !wq || !wk || !out) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (block_idx_out && !aligned16(block_idx_out)))
    return ROLA_ERR_ALIGNMENT;
  if (((uintptr_t)wq & 3u) || ((uintptr_t)wk & 3u)) return ROLA_ERR_ALIGNMENT;
  if (gate && !aligned16(gate)) return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  int32_t *map = block_idx_out ? block_idx_out : (int32_t *)(ws + P.off_map);
  ROLA_TRY(run_setup(P, wq, wk, ws, st));
  // fp8: the streaming pass also writes the scales and e4m3 tile images
  ROLA_TRY(run_pass1(P, prob, q, k, v, ws, true, true, st, P.fp8, P.vh));
  ROLA_TRY(run_reduce(P, ws, st));
  ROLA_TRY(run_select(P, ws, (float *)(ws + P.off_scores), map, st));
  return run_attn(P, prob, cfg, q, k, v, map, gate, out, ws, true, true, false, st);
}

int32_t rola_forward_train(const rola_problem *prob, const rola_config *cfg, const void *q,
                           const void *k, const void *v, const float *wq, const float *wk,
                           const float *gate, int32_t *block_idx_out, void *out, float *os, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (P.fp8) return ROLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !wq || !wk || !out || !os || !lse) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(os) ||
      (block_idx_out && !aligned16(block_idx_out)))
    return ROLA_ERR_ALIGNMENT;
  if (((uintptr_t)wq & 3u) || ((uintptr_t)wk & 3u) || ((uintptr_t)lse & 3u)) return ROLA_ERR_ALIGNMENT;
  if (gate && !aligned16(gate)) return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  int32_t *map = block_idx_out ? block_idx_out : (int32_t *)(ws + P.off_map);
  ROLA_TRY(run_setup(P, wq, wk, ws, st));
  ROLA_TRY(run_pass1(P, prob, q, k, v, ws, true, true, st, false, P.vh));
  ROLA_TRY(run_reduce(P, ws, st));
  ROLA_TRY(run_select(P, ws, (float *)(ws + P.off_scores), map, st));
  return run_attn(P, prob, cfg, q, k, v, map, gate, out, ws, true, true, false, st, lse, nullptr, os);
}

int32_t rola_forward_e4m3(const rola_problem *prob, const rola_config *cfg, const void *q,
                          const void *k, const void *v, const uint8_t *q8, const uint8_t *k8,
                          const uint8_t *v8, const float *qs, const float *ks, const float *vs,
                          const float *wq, const float *wk, const float *gate, int32_t *block_idx_out,
                          void *out, void *workspace, size_t workspace_bytes, void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (!P.fp8) return ROLA_ERR_INVALID_ARG;
  if (!q || !k || !v || !q8 || !k8 || !v8 || !qs || !ks || !vs || !wq || !wk || !out)
    return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) ||
      !aligned16(v8) || !aligned16(out) || (block_idx_out && !aligned16(block_idx_out)))
    return ROLA_ERR_ALIGNMENT;
  if (((uintptr_t)wq & 3u) || ((uintptr_t)wk & 3u) || ((uintptr_t)qs & 3u) || ((uintptr_t)ks & 3u) ||
      ((uintptr_t)vs & 3u))
    return ROLA_ERR_ALIGNMENT;
  if (gate && !aligned16(gate)) return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  int32_t *map = block_idx_out ? block_idx_out : (int32_t *)(ws + P.off_map);
  ROLA_TRY(run_setup(P, wq, wk, ws, st));
  // the streaming pass in its bf16 form (pooling and low-rank state only),
  // then the caller's codes laid out as tile images
  ROLA_TRY(run_pass1(P, prob, q, k, v, ws, true, true, st, false));
  ROLA_TRY(run_quant8(P, prob, q, k, v, ws, st, q8, k8, v8, qs, ks, vs));
  ROLA_TRY(run_reduce(P, ws, st));
  ROLA_TRY(run_select(P, ws, (float *)(ws + P.off_scores), map, st));
  return run_attn(P, prob, cfg, q, k, v, map, gate, out, ws, true, true, false, st, nullptr, q8);
}

// os, lse: the training forward's O_s and log-sum-exp (both set), or NULL:
// recompute them here
static int32_t backward_impl(const rola_problem *prob, const rola_config *cfg, const void *q,
                             const void *k, const void *v, const float *wq, const float *wk,
                             const float *gate, const int32_t *block_idx, const void *dout,
                             const float *os, const float *lse, void *dq, void *dk, void *dv, float *dwq,
                             float *dwk, float *dgate, void *workspace, size_t workspace_bytes,
                             void *stream) {
  Plan P;
  ROLA_TRY(make_plan(prob, cfg, &P));
  if (P.fp8) return ROLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !wq || !wk || !block_idx || !dout || !dq || !dk || !dv || !dwq || !dwk)
    return ROLA_ERR_INVALID_ARG;
  if ((os != nullptr) != (lse != nullptr)) return ROLA_ERR_INVALID_ARG;
  if ((os && !aligned16(os)) || ((uintptr_t)lse & 3u)) return ROLA_ERR_ALIGNMENT;
  if ((gate != nullptr) != (dgate != nullptr)) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(block_idx) || (gate && !aligned16(gate)))
    return ROLA_ERR_ALIGNMENT;
  if (((uintptr_t)wq & 3u) || ((uintptr_t)wk & 3u) || ((uintptr_t)dwq & 3u) || ((uintptr_t)dwk & 3u) ||
      ((uintptr_t)dgate & 3u))
    return ROLA_ERR_ALIGNMENT;
  if (!workspace || (int64_t)workspace_bytes < P.total_bwd) return ROLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ROLA_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  // forward state: bf16 projections, S (bf16 permuted and fp32) and z; in
  // the complement scope also the per-block states (pass 1 pools Q and K
  // along, unused) and the global sums of them
  ROLA_TRY(run_setup(P, wq, wk, ws, st));
  if (P.comp) {
    ROLA_TRY(run_pass1(P, prob, q, k, v, ws, true, true, st));
    ROLA_TRY(run_reduce(P, ws, st));
  } else {
    ROLA_TRY(run_pass1(P, prob, nullptr, k, v, ws, false, true, st));
    ROLA_TRY(timed("state_reduce", st, [&] {
      rola::launch_state_reduce((const float *)(ws + P.off_part), 2 * P.nchunks, P.D, P.r, (int)P.BH,
                                (uint16_t *)(ws + P.off_st), (float *)(ws + P.off_z),
                                (float *)(ws + P.b_s32), st);
    }));
  }
  if (os) {
    // O_s and the log-sum-exp from the training forward: only the group
    // schedule of the map is formed again
    ROLA_TRY(run_schedule(P, block_idx, ws, st));
  } else {
    // the sparse branch alone again with fp32 weights: O_s (fp32, the
    // problem's strides) and each row's log-sum-exp
    rola_config c32 = *cfg;
    c32.out_dtype = ROLA_OUT_F32;
    ROLA_TRY(run_attn(P, prob, &c32, q, k, v, block_idx, nullptr, ws + P.b_os, ws, true, false, false, st,
                      (float *)(ws + P.b_lse)));
  }
  if (P.comp) {
    // per query block: the complement state S_i, z_i (as the forward's) and
    // S_i as the hi + lo operand of the backward, on the schedule the
    // recompute left in the workspace
    rola::CompArgs ca;
    ca.blk = ws + P.off_blk;
    ca.s32 = (const float *)(ws + P.off_s32);
    ca.z = (const float *)(ws + P.off_z);
    ca.ugroup = (const int32_t *)(ws + P.off_ugroup);
    ca.ucount = (const int32_t *)(ws + P.off_ucount);
    ca.ulist = (const int32_t *)(ws + P.off_ulist);
    ca.nb = P.nb; ca.kb = P.kb;
    ca.bh_count = P.BH; ca.ngroups = P.ngroups; ca.groups_per_xcd = (P.ngroups + 7) / 8;
    ca.list_stride = P.list_stride;
    ca.stc = (uint16_t *)(ws + P.off_stc);
    ca.zc = (float *)(ws + P.off_zc);
    ca.sdc = (uint16_t *)(ws + P.b_sdc);
    ROLA_TRY(timed("complement", st, [&] { rola::launch_complement(ca, P.D, st); }));
  }

  rola::BwdArgs a;
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k; a.v = (const uint16_t *)v;
  a.dout = dout; a.dout_f32 = cfg->out_dtype == ROLA_OUT_F32;
  a.wq = wq; a.wk = wk; a.gate = gate;
  a.stride_b = prob->stride_b; a.stride_h = prob->stride_h; a.stride_n = prob->stride_n;
  a.heads = P.H; a.nb = P.nb; a.kb = P.kb; a.rank = P.r;
  a.n_tokens = P.N; a.bh_count = P.BH;
  a.scale = P.scale;
  a.scale_log2e = (float)((double)P.scale * 1.4426950408889634);
  a.rope = rope_args(P, ws);
  a.map = block_idx;
  // the recompute above left the group schedule of this map in the workspace
  a.ugroup = (const int32_t *)(ws + P.off_ugroup);
  a.ucount = (const int32_t *)(ws + P.off_ucount);
  a.ulist = (const int32_t *)(ws + P.off_ulist);
  a.ngroups = P.ngroups;
  a.groups_per_xcd = (P.ngroups + 7) / 8;
  a.list_stride = P.list_stride;
  a.wqT = (const uint16_t *)(ws + P.off_wqT); a.wkT = (const uint16_t *)(ws + P.off_wkT);
  a.st = (const uint16_t *)(ws + P.off_st);
  a.s32 = (const float *)(ws + (P.comp ? P.off_s32 : P.b_s32)); a.z = (const float *)(ws + P.off_z);
  a.os = os ? os : (const float *)(ws + P.b_os); a.lse = lse ? lse : (const float *)(ws + P.b_lse);
  a.wqP = (uint16_t *)(ws + P.b_wqP); a.wkP = (uint16_t *)(ws + P.b_wkP);
  a.sd = (uint16_t *)(ws + P.b_sd); a.dsr = (uint16_t *)(ws + P.b_dsr); a.dst = (uint16_t *)(ws + P.b_dst);
  a.ds32 = (float *)(ws + P.b_ds32); a.dz = (float *)(ws + P.b_dz);
  a.dob = (uint16_t *)(ws + P.b_dob); a.dn = (float *)(ws + P.b_dn);
  a.dqp = (float *)(ws + P.b_dqp); a.dkp = (float *)(ws + P.b_dkp); a.dvp = (float *)(ws + P.b_dvp);
  a.ahat = (uint16_t *)(ws + P.b_ahat); a.duq = (uint16_t *)(ws + P.b_duq);
  a.dwk_tok = (uint16_t *)(ws + P.b_dwk);
  a.dy = (float *)(ws + P.b_dy); a.dg = (float *)(ws + P.b_dg);
  a.part = (float *)(ws + P.b_part);
  a.tcount = (int32_t *)(ws + P.b_tcount); a.tlist = (int32_t *)(ws + P.b_tlist);
  a.tbits = (int32_t *)(ws + P.b_tbits);
  a.sumtmp = (float *)(ws + P.b_sumtmp);
  a.dq = (uint16_t *)dq; a.dk = (uint16_t *)dk; a.dv = (uint16_t *)dv;
  a.dwq = dwq; a.dwk = dwk; a.dgate = dgate;
  a.comp = P.comp ? 1 : 0;
  a.stc = P.comp ? (const uint16_t *)(ws + P.off_stc) : nullptr;
  a.zc = P.comp ? (const float *)(ws + P.off_zc) : nullptr;
  a.sdc = P.comp ? (const uint16_t *)(ws + P.b_sdc) : nullptr;
  a.pblk = P.comp ? (uint16_t *)(ws + P.b_pblk) : nullptr;
  a.dzblk = P.comp ? (float *)(ws + P.b_dzblk) : nullptr;
  a.dsrc = P.comp ? (uint16_t *)(ws + P.b_dsrc) : nullptr;
  a.dstc = P.comp ? (uint16_t *)(ws + P.b_dstc) : nullptr;
  a.dzc = P.comp ? (float *)(ws + P.b_dzc) : nullptr;
  const int D = P.D;
  ROLA_TRY(timed("bwd_prep", st, [&] { rola::launch_bwd_prep(a, D, st); }));
  ROLA_TRY(timed("bwd_query", st, [&] { rola::launch_bwd_query(a, D, st); }));
  if (P.comp) {
    // dS_i, dz_i per query block and dS per head; dz per head (and the gate
    // bias); the transposed map; then dS_j, dz_j per key block
    ROLA_TRY(timed("bwd_ds", st, [&] { rola::launch_bwd_comp_parts(a, D, st); }));
    ROLA_TRY(timed("bwd_dsops", st, [&] { rola::launch_bwd_dsops(a, D, st); }));
    ROLA_TRY(timed("bwd_tmap", st, [&] { rola::launch_bwd_tmap(a, st); }));
    ROLA_TRY(timed("bwd_dsc", st, [&] { rola::launch_bwd_comp_keys(a, D, st); }));
  } else {
    ROLA_TRY(timed("bwd_ds", st, [&] { rola::launch_bwd_outer(a, D, rola::kOuterDout, st); }));
    ROLA_TRY(timed("bwd_dsops", st, [&] { rola::launch_bwd_dsops(a, D, st); }));
  }
  ROLA_TRY(timed("bwd_key", st, [&] { rola::launch_bwd_key(a, D, st); }));
  ROLA_TRY(timed("bwd_dwq", st, [&] { rola::launch_bwd_outer(a, D, rola::kOuterRopeQ, st); }));
  ROLA_TRY(timed("bwd_dwk", st, [&] { rola::launch_bwd_outer(a, D, rola::kOuterRopeK, st); }));
  if (gate) ROLA_TRY(timed("bwd_dgate", st, [&] { rola::launch_bwd_outer(a, D, rola::kOuterGate, st); }));
  ROLA_TRY(timed("bwd_dq", st, [&] { rola::launch_bwd_dq(a, D, st); }));
  if (!P.comp) ROLA_TRY(timed("bwd_tmap", st, [&] { rola::launch_bwd_tmap(a, st); }));
  return timed("bwd_dkv", st, [&] { rola::launch_bwd_dkv(a, D, st); });
}

int32_t rola_backward(const rola_problem *prob, const rola_config *cfg, const void *q, const void *k,
                      const void *v, const float *wq, const float *wk, const float *gate,
                      const int32_t *block_idx, const void *dout, void *dq, void *dk, void *dv,
                      float *dwq, float *dwk, float *dgate, void *workspace, size_t workspace_bytes,
                      void *stream) {
  return backward_impl(prob, cfg, q, k, v, wq, wk, gate, block_idx, dout, nullptr, nullptr, dq, dk, dv, dwq,
                       dwk, dgate, workspace, workspace_bytes, stream);
}

int32_t rola_backward_saved(const rola_problem *prob, const rola_config *cfg, const void *q,
                            const void *k, const void *v, const float *wq, const float *wk,
                            const float *gate, const int32_t *block_idx, const void *dout,
                            const float *os, const float *lse, void *dq, void *dk, void *dv, float *dwq,
                            float *dwk, float *dgate, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if (!os || !lse) return ROLA_ERR_INVALID_ARG;
  return backward_impl(prob, cfg, q, k, v, wq, wk, gate, block_idx, dout, os, lse, dq, dk, dv, dwq, dwk,
                       dgate, workspace, workspace_bytes, stream);
}

int32_t rola_quant_rows(const void *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                        int64_t ld_codes, float *scale, void *stream) {
  if (!x || !codes || !scale || rows < 0 || cols <= 0 || cols % 8 || ld_x < cols || ld_x % 8 ||
      ld_codes < cols || ld_codes % 8)
    return ROLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scale & 3)) return ROLA_ERR_ALIGNMENT;
  if (rows == 0) return ROLA_OK;
  if ((rows + 3) / 4 > INT32_MAX) return ROLA_ERR_UNSUPPORTED;
  rola::QuantRowsArgs a;
  a.x = (const uint16_t *)x;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ld_x;
  a.codes = codes;
  a.ldc = ld_codes;
  a.scale = scale;
  return timed("quant_rows", (hipStream_t)stream, [&] { rola::launch_quant_rows(a, (hipStream_t)stream); });
}

int32_t rola_gemm_w8a8(const uint8_t *x, int64_t ld_x, const float *sx, const uint8_t *w,
                       int64_t ld_w, const float *sw, const float *bias, int64_t M, int32_t N,
                       int32_t K, void *out, int64_t ld_out, int32_t out_dtype, void *stream) {
  if (!x || !sx || !w || !sw || !out) return ROLA_ERR_INVALID_ARG;
  if (M < 0 || N < 4 || N % 4 || K < 64 || K % 64) return ROLA_ERR_INVALID_ARG;
  if (ld_x < K || ld_x % 16 || ld_x >= (int64_t(1) << 24) || ld_w < K || ld_w % 16 ||
      ld_w >= (int64_t(1) << 24) || ld_out < N || ld_out % 4)
    return ROLA_ERR_INVALID_ARG;
  if (out_dtype != ROLA_OUT_BF16 && out_dtype != ROLA_OUT_F32) return ROLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || !aligned16(sw) ||
      (bias && !aligned16(bias)) || ((uintptr_t)sx & 3))
    return ROLA_ERR_ALIGNMENT;
  if (M == 0) return ROLA_OK;
  const int64_t tiles_t = (M + 255) / 256, tiles_c = (N + 255) / 256;
  if (tiles_t * tiles_c > INT32_MAX) return ROLA_ERR_UNSUPPORTED;
  rola::GemmArgs a;
  a.x = x;
  a.sx = sx;
  a.w = w;
  a.sw = sw;
  a.bias = bias;
  a.out = out;
  a.M = M;
  a.ldx = ld_x;
  a.ldw = ld_w;
  a.ldo = ld_out;
  a.N = N;
  a.K = K;
  a.out_f32 = out_dtype == ROLA_OUT_F32;
  a.tiles_t = (int)tiles_t;
  a.tiles_c = (int)tiles_c;
  return timed("gemm_w8a8", (hipStream_t)stream, [&] { rola::launch_gemm_w8a8(a, (hipStream_t)stream); });
}

int32_t rola_mfma_probe(int32_t precision, int32_t iters, double *flop, float *sink, void *stream) {
  if (!flop || !sink || iters < 1) return ROLA_ERR_INVALID_ARG;
  if (precision != ROLA_PREC_BF16 && precision != ROLA_PREC_FP8) return ROLA_ERR_INVALID_ARG;
  const int blocks = 1024;  // 4 waves each: 16 waves per CU on 256 CUs
  const double per_mfma = precision == ROLA_PREC_FP8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  *flop = per_mfma * 4.0 * (double)iters * 4.0 * blocks;
  rola::launch_mfma_probe(precision == ROLA_PREC_FP8, iters, blocks, sink, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? ROLA_OK : ROLA_ERR_DEVICE;
}

int32_t rola_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing.store(on != 0);
  // create events now rather than inside the calls being timed
  while (on && g_free_events.size() < kEventPool) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) break;
    g_free_events.push_back(e);
  }
  return ROLA_OK;
}

int32_t rola_timing_read(rola_kernel_time *out, int32_t max) {
  if (!out || max < 0) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  std::vector<rola_kernel_time> agg;
  for (auto &l : g_launches) {
    float ms = 0.0f;
    if (hipEventSynchronize(l.stop) != hipSuccess) return -1;
    if (hipEventElapsedTime(&ms, l.start, l.stop) != hipSuccess) return -1;
    g_free_events.push_back(l.start);
    g_free_events.push_back(l.stop);
    bool found = false;
    for (auto &a : agg) {
      if (l.name == a.name) {
        a.launches += 1;
        a.total_ms += ms;
        found = true;
        break;
      }
    }
    if (!found) {
      rola_kernel_time t;
      std::memset(&t, 0, sizeof t);
      std::strncpy(t.name, l.name.c_str(), sizeof t.name - 1);
      t.launches = 1;
      t.total_ms = ms;
      agg.push_back(t);
    }
  }
  g_launches.clear();
  int32_t n = 0;
  for (auto &a : agg) {
    if (n >= max) break;
    out[n++] = a;
  }
  return n;
}

}  // extern "C"
