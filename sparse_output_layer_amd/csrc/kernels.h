// kernels.h -- launchers of the gfx950 kernels (internal C++ interface of
// libhaste; the public interface is include/haste.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace haste {

// Everything a tail kernel may read or write.  Pointers not used by a
// given launch may be null.
struct TailArgs {
    const unsigned short *XT;    // D x Bp bf16, zero beyond column B
    const int32_t *idx;          // Ng x F
    const unsigned short *W;     // (Ng*G) x F bf16
    unsigned short *Z;           // B x L bf16 (forward output)
    const unsigned short *dZ;    // B x L bf16 (given gradient)
    float *Z32;                  // fp32 logits for the top-K: B x L, row stride L; or null
    float *tk_v;                 // fused top-K stage 1 (one bucket per group, K' = 1): Ng x Bp
    int32_t *tk_i;               //   largest logit of each (group, row) and its id (-1: none); or null
    int64_t tk_off;              //   id of tail label 0
    int tk_max_only;             //   1: each list entry's id is its group's first label (the exact
                                 //   top-K needs only the groups); 0: the maximum's own id
    const unsigned short *idxp;  // Ng x F: idx in T1's bank-aware order (idxp[g][k] = idx[g][perm[g][k]])
    const unsigned char *perm;   // Ng x F: that order's feature per position
    unsigned short *dzt;         // dz tiles of the dW pass for the dX pass, or null:
                                 // Ng x (Bp/32) x (G/16) tiles of 1 KB (32 rows x 16 labels)
    unsigned short *dW;          // (Ng*G) x F bf16, or null when Wout is set
    unsigned short *Wout;        // (Ng*G) x F bf16: W - lr * dW (fused SGD), or null
    float lr;                    // SGD step of Wout
    float *dX;                   // B x D fp32 (atomically accumulated)
    const int32_t *grp_ptr;      // Ng + 1 group-major positives
    const int32_t *grp_ent;      // entries b*G + j
    float *loss;                 // fp32 scalar (+=)
    float s;                     // gradient scale
    unsigned *sched;             // 2 counters of the dW/logits pass's dynamic run order (zero
                                 //   between launches: the prep zeroes them, the pass's last
                                 //   workgroup resets them)
    int B, D, Bp, F;
    int64_t L, Ng;
};

enum T1Mode { T1_FWD = 0, T1_DW_BCE = 1, T1_DW_MEM = 2 };

// Launch helpers return hipSuccess or the launch error.
hipError_t launch_transpose_x(const unsigned short *X, unsigned short *XT, int B, int D, int Bp,
                              unsigned *sched, hipStream_t st);
hipError_t launch_fill_u32(void *p, uint32_t v, size_t n, hipStream_t st);
// out = W - lr * dW elementwise (bf16 or fp32 by `bf16`), n elements
hipError_t launch_sgd(const void *W, const void *dW, float lr, void *out, int64_t n, bool bf16,
                      hipStream_t st);
hipError_t launch_feature_order(const int32_t *idx, int64_t Ng, int F, unsigned short *idxp,
                                unsigned char *perm, hipStream_t st);
hipError_t launch_group_positives(const int32_t *row_ptr, const int32_t *labels,
                                  int nnz, int B, int64_t label_offset,
                                  int64_t L, int G, int64_t Ng, long long *keys,
                                  int32_t *grp_ptr, int32_t *ent,
                                  hipStream_t st);
hipError_t launch_tail_t1(int mode, int G, const TailArgs &a, bool store_z,
                          bool do_loss, hipStream_t st);
// dz_mode: 0 recompute dz from the positives, 1 read the B x L dZ,
// 2 read the dz tiles (dzt) that the dW pass (T1_DW_BCE) stored
hipError_t launch_tail_t2(int G, int dz_mode, const TailArgs &a,
                          hipStream_t st);
bool tail_bf16_supported(int G, int F, int D);
// dX from the stored dz tiles at the layer's own flops (Y_g = dz_g W_g, then a
// scatter into an LDS-resident dX^T tile of 32 rows): shapes it takes, launch
bool tail_dxs_supported(int G, int F, int D);
hipError_t launch_tail_dxs(int G, const TailArgs &a, hipStream_t st);
// G = 1 (per-label fan-in): logits and loss only
hipError_t launch_fanin1_fwd(const TailArgs &a, bool store_z, bool do_loss, hipStream_t st);
// G = 1 training step: logits, loss, dz (label-major into dzt, L x Bp bf16),
// dW, then dX from dzt; shapes it takes (F in {32, 64, 128}, 16 <= D <= 960)
bool fanin1_step_supported(int F, int D);
hipError_t launch_fanin1_step(const TailArgs &a, bool do_loss, hipStream_t st);

// Per-row top-K (K in [1, 8]) of fp32 logits z (rows x n, row stride ld,
// column c has id id_offset + c): stage 1 keeps the top-KP (1 <= KP <= K;
// 0 means K) of every bucket into cand (rows x nseg x KP), stage 2 merges
// them into out (rows x K).  Buckets: nbuckets runs of ceil(n / nbuckets)
// consecutive columns; nbuckets == 0 -> about TOPK_WG / rows of them.
constexpr int64_t TOPK_WG = 1024;
struct TopkBuckets {
    int64_t seg_len, nseg;
};
TopkBuckets topk_buckets(int64_t n, int64_t nbuckets, int64_t rows);
hipError_t launch_row_topk(const float *z, int64_t ld, int rows, int64_t n, int64_t id_offset,
                           int K, int KP, int64_t nbuckets, float *cand_v, int32_t *cand_i,
                           float *out_v, int32_t *out_i, hipStream_t st);
// stage 2 alone over rows x ncand candidates
hipError_t launch_topk_merge_cands(const float *cand_v, const int32_t *cand_i, int rows,
                                   int64_t ncand, int K, float *out_v, int32_t *out_i,
                                   hipStream_t st);
// Merge of group-major candidates (ngroups x ld, row-contiguous; stage 1 fused
// into the logits pass): segments of groups per block of rows into mid
// (rows x nseg x K), then per row into out (rows x K)
constexpr int64_t TOPK_GM_BLOCKS = 512;
struct TopkGmSegs {
    int64_t seg_groups, nseg;
};
TopkGmSegs topk_gm_segments(int64_t ngroups, int64_t rows);
hipError_t launch_topk_group_major(const float *gv, const int32_t *gi, int64_t ld, int rows,
                                   int64_t ngroups, int K, float *mid_v, int32_t *mid_i,
                                   float *out_v, int32_t *out_i, hipStream_t st);

// Exact top-K from the K best groups of each row (out_i: their maxima's ids,
// from launch_topk_group_major): the groups' logits recomputed bit for bit
// as the logits pass forms them (bf16 X row-major, W, the feature order
// idxp / perm), the K best kept, in place in out_v / out_i
hipError_t launch_topk_refine(const unsigned short *X, int B, int D, const unsigned short *W,
                              const unsigned short *idxp, const unsigned char *perm, int G, int F,
                              int64_t L, int64_t tk_off, int K, float *out_v, int32_t *out_i,
                              hipStream_t st);

// One prune-and-regrow step of every group's fan-in set: shapes it takes
// (G <= 64, F <= 256, F <= D <= 65536); idx_out / W_out may be idx / W
bool rewire_supported(int G, int F, int D);
hipError_t launch_rewire(const int32_t *idx, const void *W, bool bf16, int64_t Ng, int G, int F,
                         int D, int64_t L, int k, const int32_t *cand, int R, int32_t *idx_out,
                         void *W_out, hipStream_t st);

// A caller's dZ (B x L bf16, row-major) into the dW pass's dz tiles
hipError_t launch_dz_tiles(const unsigned short *dZ, int B, int64_t L, int G, int Bp, int64_t Ng,
                           unsigned short *dzt, hipStream_t st);

// Measurement utility: blocks x 4 waves, iters rounds of 16 independent
// 16x16x32 bf16 MFMAs each (no memory traffic)
hipError_t launch_probe_mfma(int blocks, int iters, float *sink, hipStream_t st);

// Head (dense classifier) GEMMs.
struct GemmArgs {
    const unsigned short *A;
    const unsigned short *Bm;
    int M, N, K;
    int lda, ldb;              // row strides (elements)
    // epilogue
    unsigned short *C16;       // bf16 output, ldc = N
    float *C32;                // fp32 output (atomic add), ldc = N
    unsigned short *Zout;      // BCE: optional logits (bf16), ld N
    unsigned short *dZout;     // BCE: optional dz (bf16), ld N
    float *Z32;                // BCE: optional fp32 logits (for the top-K), ld N
    const uint32_t *bitmap;    // BCE: positives bitmap, row stride bm_words
    int bm_words;
    const int32_t *pos_ptr;    // BCE on the pipelined GEMM (gemm2_shape): the positives as
    const int32_t *pos_lab;    //   row CSR, global ids, column c = id - pos_off (instead of
    int64_t pos_off;           //   the bitmap; read per tile in the GEMM's prologue)
    int pos_nnz;               //   entries of pos_lab (reads stay below it)
    float *loss;
    float s;
    int k_split;               // K elements per split (multiple of 32)
};
enum GemmEpi { EPI_BCE = 0, EPI_STORE16 = 1, EPI_ATOMIC32 = 2 };
// a_kmaj: A stored [m][k]; else [k][m].  b_kmaj: B stored [n][k]; else [k][n].
hipError_t launch_gemm(bool a_kmaj, bool b_kmaj, int epi, const GemmArgs &g,
                       hipStream_t st);
// the pipelined GEMM takes the shape (M, N, K and the split multiples of 8)
bool gemm2_shape(const GemmArgs &g);
hipError_t launch_head_bitmap(const int32_t *row_ptr, const int32_t *labels,
                              int nnz, int B, int64_t label_offset, int H,
                              uint32_t *bm, int bm_words, hipStream_t st);

// fp32 (VALU) path.
struct F32Args {
    const float *X;
    const int32_t *idx;
    const float *W;
    float *Z;
    float *dZ;                 // given or workspace
    float *dW;
    float *dX;
    const int32_t *row_ptr;
    const int32_t *labels;
    int64_t label_offset;
    float *loss;
    float s;
    int B, D, G, F;
    int64_t L, Ng;
};
hipError_t launch_f32_tail_logits(const F32Args &a, bool store_z, bool bce,
                                  bool loss, hipStream_t st);
hipError_t launch_f32_tail_dw(const F32Args &a, hipStream_t st);
hipError_t launch_f32_tail_dx(const F32Args &a, hipStream_t st);
hipError_t launch_f32_head_logits(const F32Args &a, bool store_z, bool bce,
                                  bool loss, hipStream_t st);
hipError_t launch_f32_head_dw(const F32Args &a, hipStream_t st);
hipError_t launch_f32_head_dx(const F32Args &a, hipStream_t st);

// utilities
hipError_t launch_validate(const int32_t *idx, int64_t Ng, int F, int D,
                           int32_t *first_bad, hipStream_t st);
hipError_t launch_topk_merge(int B, int K, const float *av, const int32_t *ai,
                             const float *bv, const int32_t *bi, float *ov,
                             int32_t *oi, hipStream_t st);

}  // namespace haste
