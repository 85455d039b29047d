// rola_internal.h -- argument blocks shared by the librola host code and its kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rola {

struct RopeArgsHost {
  int off1, off2;           // first dims of the h and w axes
  int half0, half1, half2;  // rotary pairs per axis
  int grid_h, grid_w;
  float log2_theta;
};

struct SetupArgs {
  const float *wq, *wk;
  int D, rank;
  uint16_t *wqT, *wkT;  // bf16 [32][D]
};

struct Pass1Args {
  const uint16_t *q, *k, *v;
  int64_t stride_b, stride_h, stride_n;
  int heads;
  int nb;
  int64_t n_tokens;
  int cpc;              // 64-token blocks per workgroup
  int rank;
  float inv_tail;       // fl32(1/valid) of the tail block
  float *qp, *kp;       // pooled [BH][nb][D]
  const uint16_t *wkT;  // bf16 [32][D]
  float *state_part;    // [BH][nchunks][2][D*32 + 32]
  uint8_t *blk_state;   // complement scope: [BH][nb] per-block states (bf16 S^T [D][32], fp32 z
                        // [32]; D*64 + 128 bytes each), else NULL
  RopeArgsHost rope;
  // fp8 mode (see Quant8Args): Q scales, K and V^T codes of each block
  float *qsc, *ksc, *vsc;
  uint8_t *kv8;
  // fp16 copy of V (bf16 output), written by the pooling waves: [BH][n_pad][D]
  // (rows past N not written), and two range flags per (batch*head, chunk),
  // [BH][2 * gridDim.x]: 1 if a valid |v| of the chunk's half is >= 2^16 (or
  // inf), beyond fp16, else 0 -- all written on every pass, so never cleared
  uint16_t *vh;
  int32_t *vovf;
};

// Attention workgroup shape: G query blocks per workgroup (2 waves each),
// S-slot LDS ring of K/V^T tiles.
constexpr int kAttnG = 4;
constexpr int kAttnS = 4;


// fp8 copies of the token tensors (k_quant8): per (batch, head, block)
// scales and one tile image of e4m3 K and V^T codes per block.
struct Quant8Args {
  const uint16_t *q, *k, *v;
  int64_t stride_b, stride_h, stride_n;
  int heads, nb;
  int64_t n_tokens;
  // pre-quantised input (else NULL): e4m3 codes with the strides of q, k, v
  // (in elements) and their per-block scales [BH][nb]; the kernel then only
  // lays the codes out as tile images and copies the scales
  const uint8_t *q8, *k8, *v8;
  const float *qs_in, *ks_in, *vs_in;
  float *qsc;     // [BH][nb][2]: fl32(absmax/448), fl32(448/absmax) of Q
  float *ksc;     // [BH][nb]: fl32(absmax/448) of K
  float *vsc;     // [BH][nb]: fl32(absmax/448) of V
  uint8_t *kv8;   // [BH][nb][64*D] K tile images (e4m3 codes)
  uint16_t *vh;   // [BH][n_pad][D] the V codes as fp16 values (exact), rows past N zero
};

// fp8 attention: ring depth (24 KB tiles at D=128), tiles per barrier and
// union-list entries staged in LDS
constexpr int kAttn8S = 4;
constexpr int kAttn8P = 2;
constexpr int kAttn8Lmax = 1024;

struct AttnArgs {
  const uint16_t *q, *k, *v;
  void *out;
  int64_t stride_b, stride_h, stride_n;
  int heads, nb, kb, rank;
  int64_t n_tokens;
  int64_t bh_count;
  int64_t ngroups;         // groups of G query blocks per (batch, head)
  int64_t groups_per_xcd;  // ceil(ngroups / 8)
  int64_t list_stride;     // G * kb
  const int32_t *ugroup;   // [BH][ngroups][G] member query blocks (-1: none)
  const int32_t *ucount;   // [BH][ngroups] union length
  const int32_t *ulist;    // [BH][ngroups][list_stride] key block | member mask << 16
  float scale_log2e;
  const uint16_t *wqT;  // bf16 [32][D]
  const uint16_t *st;   // bf16 [BH][D][32] (rank permuted)
  const float *z;       // [BH][32]
  const uint16_t *vh;   // fp16 V copy and its range flags (see Pass1Args), bf16 output
  const int32_t *vovf;  // with the sparse branch; nflags flags per (batch, head)
  int nflags;
  const float *gate;    // fp32 [D+1] output gate (w, then b) on the low-rank term; NULL: none
  int complement;       // st and z hold one state per query block ([BH][nb][D][32], [BH][nb][32])
  float *lse;           // if set, the base-2 log-sum-exp of each row's scaled logits
                        // (s * scale * log2 e), [BH][n_pad]: the backward's recompute (the
                        // sparse branch alone, fp32 weights) or the training forward
  float *os_save;       // training forward (fused, bf16 operands): if set, the sparse
                        // branch's output O_s, fp32 with the problem's strides (rows >= N 0)
  RopeArgsHost rope;
  // fp8 sparse branch only
  const uint8_t *kv8;   // tile images, see Quant8Args
  const float *qsc, *ksc, *vsc;
  const uint8_t *q8;    // fp8 with pre-quantised input: Q codes (strides of q), else NULL
};

void launch_setup(const SetupArgs &a, hipStream_t st);
// per-block states as well when a.blk_state is set; the fp16 V copy when
// a.vh is set (not with quant; with neither pool nor state: the copy alone)
void launch_pass1(const Pass1Args &a, int D, int nchunks, int bh, bool pool, bool state, bool quant,
                  hipStream_t st);
// part: np fp32 partial states per head, [BH][np][D*32 + 32]
void launch_state_reduce(const float *part, int np, int D, int rank, int bh, uint16_t *st_out,
                         float *z, float *s32, hipStream_t st);
// complement scope: `parts` block-range sums of pass 1's per-block states into
// part ([BH][parts][D*32 + 32]) for launch_state_reduce
void launch_blk_partial(const uint8_t *blk, int nb, int parts, int D, int bh, float *part, hipStream_t st);

// Complement scope: per query block, the global state minus the states of its
// kept key blocks, gathered along the attention schedule's union lists.
struct CompArgs {
  const uint8_t *blk;      // [BH][nb] per-block states as written by pass 1 (bf16 S^T, fp32 z)
  const float *s32, *z;    // global S [BH][D*32] and z [BH][32]
  const int32_t *ugroup, *ucount, *ulist;
  int nb, kb;
  int64_t bh_count, ngroups, groups_per_xcd, list_stride;
  uint16_t *stc;           // out: bf16 [BH][nb][D][32], rank-permuted like st
  float *zc;               // out: [BH][nb][32]
  uint16_t *sdc;           // out (backward only, else NULL): bf16 [2][BH][nb][32][D], the
                           // complement S with d permuted per 16-group, as hi + lo (like sd)
};
void launch_complement(const CompArgs &a, int D, hipStream_t st);
void launch_scores(const float *qp, const float *kp, float *s, int nb, int D, int bh,
                   hipStream_t st);
void launch_topk(const float *s, int32_t *map, int nb, int kb, int64_t rows, hipStream_t st);
void launch_schedule(const int32_t *map, int nb, int kb, int G, int ngroups, int list_stride,
                     int bh, int32_t *ugroup, int32_t *ucount, int32_t *ulist, hipStream_t st);
int attn_group_size();
void launch_attn(const AttnArgs &a, int D, bool sparse, bool lowrank, bool accum, bool outf32,
                 hipStream_t st);
void launch_quant8(const Quant8Args &a, int D, int bh, hipStream_t st);
void launch_mfma_probe(bool fp8, int iters, int blocks, float *sink, hipStream_t st);
void launch_attn8(const AttnArgs &a, int D, bool lowrank, bool accum, bool outf32, hipStream_t st);

// ---------------------------------------------------------------- backward
// Buffers of one rola_backward call.  Token-major work arrays are [BH][n_pad]
// rows; bf16 arrays hold uint16 bit patterns.
struct BwdArgs {
  // inputs (caller layout for q, k, v, dout; strides in elements)
  const uint16_t *q, *k, *v;
  const void *dout;  // bf16 or fp32 (dout_f32)
  int dout_f32;
  const float *wq, *wk, *gate;
  int64_t stride_b, stride_h, stride_n;
  int heads, nb, kb, rank;
  int64_t n_tokens, bh_count;
  float scale, scale_log2e;
  RopeArgsHost rope;
  const int32_t *map;  // [BH][nb][kb], ascending
  // the forward's group schedule of the same map (see AttnArgs), or NULL
  const int32_t *ugroup, *ucount, *ulist;
  int64_t ngroups, groups_per_xcd, list_stride;
  // state of the forward (from pass 1 and the reduction)
  const uint16_t *wqT, *wkT;  // bf16 [32][D]
  const uint16_t *st;         // bf16 [BH][D][32], rank-permuted
  const float *s32, *z;       // S^T fp32 [BH][D][32], z [BH][32]
  const float *os;            // recomputed sparse output, fp32, the problem's strides
  const float *lse;           // [BH][n_pad], base 2, from the recompute
  // operand copies
  uint16_t *wqP, *wkP;        // bf16 [D][32], rank-permuted
  uint16_t *sd;               // bf16 [2][BH][32][D], S with d permuted per 16-group (hi, lo)
  uint16_t *dsr;              // bf16 [BH][32][D], dS (natural)
  uint16_t *dst;              // bf16 [BH][D][32], dS^T rank-permuted
  float *ds32;                // fp32 [BH][D][32], dS^T
  float *dz;                  // [BH][32]
  // per-token work arrays
  uint16_t *dob;              // dO in bf16 [BH][n_pad][D] (0 on padded rows)
  float *dn;                  // D_n = dO_n . O_s,n [BH][n_pad]
  float *dqp, *dkp, *dvp;     // low-rank and gate parts of dq, dk, dv, fp32 [BH][n_pad][D]
  uint16_t *ahat, *duq, *dwk_tok;  // bf16 [BH][n_pad][32]: g a / den, dL/du (query), dL/dw (key)
  float *dy, *dg;             // gate: dL/d(q.w + b), dL/dg [BH][n_pad]
  float *part;                // reduction partials
  float *sumtmp;              // per-head sums of the pooled gradients [BH][D][32]
  int32_t *tcount, *tlist;    // query blocks keeping each key block: [BH][nb], [BH][nb][nb]
  int32_t *tbits;             // the map as bitsets over key blocks [BH][nb][ceil(nb/32)]
  // complement scope (comp != 0): per query block i the state S_i, z_i over
  // the key blocks i does not keep (from the forward's complement kernel),
  // and per key block j the gradient of its block state, dS_j = sum over the
  // query blocks that do not keep j of their dS_i
  int comp;
  const uint16_t *stc;        // bf16 [BH][nb][D][32], rank-permuted (as st)
  const float *zc;            // [BH][nb][32]
  const uint16_t *sdc;        // bf16 [2][BH][nb][32][D], d permuted (as sd: hi, lo)
  uint16_t *pblk;             // bf16 [BH][nb][D][32]: dS_i^T per query block
  float *dzblk;               // [BH][nb][32]: dz_i per query block
  uint16_t *dsrc, *dstc;      // bf16 [BH][nb][32][D] (as dsr), [BH][nb][D][32] (as dst): dS_j
  float *dzc;                 // [BH][nb][32]: dz_j
  // outputs
  uint16_t *dq, *dk, *dv;     // bf16, caller layout
  float *dwq, *dwk, *dgate;   // [D][rank], [D][rank], [D+1]
};

// X^T Y reductions over tokens (dWq, dWk, dS, gate weights)
enum BwdOuterMode { kOuterRopeQ = 0, kOuterDout = 1, kOuterRopeK = 2, kOuterGate = 3, kOuterDoutBlk = 4 };

void launch_bwd_prep(const BwdArgs &a, int D, hipStream_t st);   // wqP, wkP, sd
void launch_bwd_query(const BwdArgs &a, int D, hipStream_t st);  // low-rank and gate, per query token
void launch_bwd_outer(const BwdArgs &a, int D, int mode, hipStream_t st);
void launch_bwd_dsops(const BwdArgs &a, int D, hipStream_t st);  // dz, then dS operands
void launch_bwd_key(const BwdArgs &a, int D, hipStream_t st);    // low-rank, per key token
// complement scope: dS_i, dz_i per query block and their head totals, then
// (after the transposed map) dS_j, dz_j per key block as operand copies
void launch_bwd_comp_parts(const BwdArgs &a, int D, hipStream_t st);
void launch_bwd_comp_keys(const BwdArgs &a, int D, hipStream_t st);
void launch_bwd_dq(const BwdArgs &a, int D, hipStream_t st);     // sparse dq (+ the low-rank part)
void launch_bwd_tmap(const BwdArgs &a, hipStream_t st);
void launch_bwd_dkv(const BwdArgs &a, int D, hipStream_t st);    // sparse dk, dv (+ low-rank parts)
int bwd_outer_parts(int64_t bh_count, int nb, int mode);        // partials written per mode

// w8a8 linear layers
struct QuantRowsArgs {
  const uint16_t *x;  // bf16 [rows, cols], row stride ldx (elements)
  int64_t rows, cols, ldx;
  uint8_t *codes;     // e4m3 [rows, cols], row stride ldc (bytes)
  int64_t ldc;
  float *scale;       // [rows]
};
struct GemmArgs {
  const uint8_t *x;   // e4m3 activations [M, K], row stride ldx
  const float *sx;    // [M]
  const uint8_t *w;   // e4m3 weights [N, K], row stride ldw
  const float *sw;    // [N]
  const float *bias;  // [N] or null
  void *out;          // [M, N] bf16 or fp32, row stride ldo (elements)
  int64_t M, ldx, ldw, ldo;
  int N, K, out_f32;
  int tiles_t, tiles_c;
};
void launch_quant_rows(const QuantRowsArgs &a, hipStream_t st);
void launch_gemm_w8a8(const GemmArgs &a, hipStream_t st);

}  // namespace rola
