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
};

// Attention workgroup shape: G query blocks per workgroup (2 waves each),
// S-slot LDS ring of K/V^T tiles.
#ifndef ROLA_ATTN_G
#define ROLA_ATTN_G 4
#endif
#ifndef ROLA_ATTN_S
#define ROLA_ATTN_S 4
#endif


// fp8 copies of the token tensors (k_quant8): per (batch, head, block)
// scales and one tile image of e4m3 K and V^T codes per block.
struct Quant8Args {
  const uint16_t *q, *k, *v;
  int64_t stride_b, stride_h, stride_n;
  int heads, nb;
  int64_t n_tokens;
  float *qsc;     // [BH][nb][2]: fl32(absmax/448), fl32(448/absmax) of Q
  float *ksc;     // [BH][nb]: fl32(absmax/448) of K
  float *vsc;     // [BH][nb]: fl32(absmax/448) of V
  uint8_t *kv8;   // [BH][nb][128*D] tile images (K rows, then V^T rows)
};

// fp8 attention: ring depth (16 KB tiles at D=128), tiles per barrier and
// union-list entries staged in LDS
#ifndef ROLA_ATTN8_S
#define ROLA_ATTN8_S 8
#endif
#ifndef ROLA_ATTN8_P
#define ROLA_ATTN8_P 4
#endif
#ifndef ROLA_ATTN8_LMAX
#define ROLA_ATTN8_LMAX 1024
#endif

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
  const float *gate;    // fp32 [D+1] output gate (w, then b) on the low-rank term; NULL: none
  int complement;       // st and z hold one state per query block ([BH][nb][D][32], [BH][nb][32])
  RopeArgsHost rope;
  // fp8 sparse branch only
  const uint8_t *kv8;   // tile images, see Quant8Args
  const float *qsc, *ksc, *vsc;
};

void launch_setup(const SetupArgs &a, hipStream_t st);
void launch_pass1(const Pass1Args &a, int D, int nchunks, int bh, bool pool, bool state, bool quant,
                  hipStream_t st);  // per-block states as well when a.blk_state is set
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

}  // namespace rola
