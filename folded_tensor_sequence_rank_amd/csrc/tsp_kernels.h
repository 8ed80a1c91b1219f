// Internal launch interface between the C ABI (tsp_api.cpp) and the gfx950
// kernels (tsp_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsp {

enum Dtype { BF16 = 0, F32 = 1 };

// Epilogues of the projection GEMM C = A . B^T (A [M][K], B [N][K]).
enum Epi {
  EPI_ACC = 1,    // Y = (beta ? Y : 0) + acc            (fp32 accumulator, in place)
  EPI_RESID = 2,  // C = R + (beta ? Y : 0) + acc         (residual add, output dtype)
  EPI_QKV = 3,    // scatter columns to Q / K / Vt at zigzag positions
  EPI_SWIGLU = 4,  // C = silu(A.B1^T) * (A.B3^T)          (two B operands)
  EPI_STORE = 5,   // C = acc                               (output dtype)
  // EPI_QKV with the rotary embedding (rope_l2 > 0): launch_gemm picks it for
  // EPI_QKV calls that rotate, so the plain instance carries no fp64 angle code
  EPI_QKV_ROPE = 6
};

struct GemmArgs {
  const void* A;
  const void* B;
  const void* B3;  // second B operand (EPI_SWIGLU)
  // EPI_SWIGLU over two weight blocks: output columns from n_split on take
  // their W1 / W3 rows from B_2 / B3_2 (row c - n_split) instead of B / B3
  // (n_split = 0: one block).
  const void* B_2;
  const void* B3_2;
  int n_split;
  int64_t lda, ldb;
  int M, N, K;
  void* C;
  int64_t ldc;
  float* Y;
  int64_t ldy;
  int beta;
  const void* R;
  int64_t ldr;
  // EPI_QKV: column c (after adding col0) is Q for c < hs (head c / hd, dim
  // c % hd), then K for ks columns and V for ks columns (K/V head
  // (c - hs) % ks / hd).  With B = batch sequences (0 means 1) of length S and
  // T local rows each, Q is [heads][B*T][hd], K is [kv heads][B*S][hd] and Vt
  // is [kv heads][hd][B*S]; local row m = b*T + i of sequence b sits at row
  // b*S + zigzag(i).  rope_l2 = log2(theta) > 0 rotates Q and K at the row's
  // position in its sequence (0: no rotation).
  // Several shards in one launch (shard_cols > 0): column c belongs to shard
  // c / shard_cols, whose Q, K and Vt start q_stride and kv_stride elements
  // further on per shard.
  void* Q;
  void* Kd;
  void* Vt;
  int hs, ks, hd, col0;
  int shard_cols;
  int64_t q_stride, kv_stride;
  double rope_l2;
  int64_t S, T;
  int64_t chunk;
  int rank, fold;
  int batch;
};

// B = batch sequences; T local rows and S positions per sequence.
struct AttnArgs {
  const void* Q;   // [Hd][B*T][HD]
  const void* K;   // [Hd/grp][B*S][HD]
  const void* Vt;  // [Hd/grp][HD][B*S]
  // Other ranks' rows read in place (same layouts as K / Vt), or null when K
  // and Vt hold every row.  With them, K and Vt are read only in the rank's
  // own chunks, and chunk boundaries fall on 64-key tile boundaries.
  const void* Kg;
  const void* Vtg;
  void* O;         // [B*T][ldo]; head t writes columns [t*HD, (t+1)*HD)
  float* Op;       // partial outputs of split items [Hd][B][nqt][maxseg][bq][HD]
  float* ML;       // partial (max, sum) [Hd][B][nqt][maxseg][bq][2]
  float* LSE;      // optional: per row log2 of its softmax normaliser, [Hd][B*T]
  int64_t T, S, chunk;
  int ldo, rank, fold, Hd;
  int batch;
  int grp;  // query heads per K/V head (0 means 1)
  // Several shards in one launch (kvh_per_shard > 0): K/V head kvh is head
  // kvh % kvh_per_shard of shard kvh / kvh_per_shard, whose K, Vt, Kg and Vtg
  // blocks start shard_stride elements further on per shard.
  int kvh_per_shard;
  int64_t shard_stride;
  int bq, nqt, lseg, maxseg, nitems;  // bq: local query rows per tile (the plan's)
  float scale_log2;  // log2(e) / sqrt(HD)
  float sum_cap;     // largest 32-key block sum of exponentials before the reference max is raised
};

// Attention work plan for one head group (a deterministic function of the dims).
struct AttnPlan {
  int bq;      // local query rows per tile
  int nqt;     // query tiles of bq local rows
  int lseg;    // keys per split item (multiple of 64)
  int maxseg;  // largest number of splits of one query tile
  int nitems;  // work items per head
  bool split;  // any query tile has more than one split
};
// wide: the 256-row query tiles of the bf16 128-dim kernel (one workgroup
// per CU), else 128-row tiles (two per CU).
AttnPlan attn_plan(int64_t T, int64_t S, int64_t chunk, int rank, int fold, int Hd, bool wide);
// Whether attention of this dtype and head dim runs on 256-row query tiles.
bool attn_wide(Dtype dt, int hd);

hipError_t launch_rmsnorm(Dtype dt, const void* x, const void* g, void* y, int64_t rows, int h,
                          float eps, hipStream_t s);
hipError_t launch_gemm(Dtype dt, Epi epi, const GemmArgs& a, hipStream_t s);
// part 0: the attention kernel; part 1: the merge of split items (no-op
// when the plan has no split).
hipError_t launch_attention(Dtype dt, int head_dim, const AttnArgs& a, const AttnPlan& p,
                            int part, hipStream_t s);
hipError_t launch_fill32(void* p, uint32_t pattern, size_t bytes, hipStream_t s);
hipError_t launch_spin(uint64_t ticks, hipStream_t s);
// n (wall-clock tick, shader-clock cycle) pairs into out[2n], one every
// `interval` wall-clock ticks (n * interval is bounded by the caller).
hipError_t launch_clock_probe(uint64_t* out, int n, uint64_t interval, hipStream_t s);
// Backward of the MLP half.
hipError_t launch_transpose(Dtype dt, const void* in, void* out, int64_t R, int64_t C, int64_t ldi,
                            int64_t ldo, hipStream_t s);
// Batched transpose into a row-padded layout: for z in [0, Z), r in [0, Rp),
// c in [0, C): out[c * ldo + z * Rp + r] = r < R ? in[zoff + r * ldi + c] : 0,
// zoff = (z / zdiv) * s1 + (z % zdiv) * s0.  Rp is a multiple of 64.
hipError_t launch_transpose_pad(Dtype dt, const void* in, void* out, int64_t R, int64_t Rp, int64_t C,
                                int64_t ldi, int64_t ldo, int64_t Z, int64_t zdiv, int64_t s1, int64_t s0,
                                hipStream_t s);
// ab: [rows][2F] fp32, a = n W1 then b = n W3; dg: [rows][F] fp32.
hipError_t launch_swiglu_bwd(Dtype dt, const float* ab, const float* dg, void* dab, void* g, int64_t rows,
                             int64_t F, hipStream_t s);
// dx = res + RMSNorm'(x)^T dn; dgain += the gain's gradient (not zeroed here),
// summed in a fixed order through partial (gain_partial_floats(rows, h)
// floats of scratch).
hipError_t launch_rmsnorm_bwd(Dtype dt, const void* x, const void* g, const float* dn, const void* res,
                              void* dx, float* rs, float* dgain, float* partial, int64_t rows, int h, float eps,
                              hipStream_t s);
int64_t gain_partial_floats(int64_t rows, int h);

// Rotations undone: every 4-dim group of v (fp32, rows of hd values, `rows`
// rows per head, `heads` heads) turned back by its row's position.  Row m of
// a head is position m % S of its sequence when S > 0 (gathered K/V rows), or
// the zigzag position zig(m % T) when S == 0 (local rows).  l2c = log2(theta)/hd.
hipError_t launch_rope_inverse(float* v, int64_t rows, int heads, int hd, int64_t S, int64_t T, int64_t chunk,
                               int rank, int fold, double l2c, hipStream_t s);
// own[j][c][t][b*T + i][e] = sum over the D ranks' partials part[q][j][c][t][b*S + zig(i)][e]
// (j < D shards, c: K or V, t < hkd heads, e < hd): the sums a reduce-scatter of
// per-position gradients delivers to rank `rank`, gathered at its local rows.
constexpr int kMaxFold = 64;
struct KvGradReduceArgs {
  const float* part[kMaxFold];
  float* own;
  int64_t S, T, chunk, batch;
  int rank, fold, hkd, hd;
};
hipError_t launch_kv_grad_reduce(const KvGradReduceArgs& a, hipStream_t s);
// out[m][c] (row pitch hs + 2ks) from dq [hd-dim heads][rows][hd] for c < hs,
// dk [..][rows][hd] for the next ks columns and dv for the last ks.
hipError_t launch_qkv_grad_pack(Dtype dt, const float* dq, const float* dk, const float* dv, void* out,
                                int64_t rows, int hs, int ks, int hd, hipStream_t s);

// Backward of the attention core (bf16, head dim 64 or 128).
struct AttnBwdArgs {
  const void* Q;     // [Hd][B*T][HD] rotated queries
  const void* K;     // [Hkd][B*S][HD]
  const void* Vt;    // [Hkd][HD][B*S]
  const void* O;     // [B*T][ldo_fwd] forward output, head t at columns t*HD
  const void* dO;    // [B*T][ldo] its gradient, the same columns
  const float* LSE;  // [Hd][B*T] log2 of each row's softmax normaliser (scaled scores)
  float* Dl;         // [Hd][B*T] rowsum(dO * O)
  float* dQ;         // [Hd][B*T][HD]
  float* dQp;        // [Hd][B][dq_items][128][HD]: partial dQ of each (query block, key segment) item
  float* dK;         // [Hkd][B*S][HD]
  float* dV;         // [Hkd][B*S][HD]
  const void* Qt;    // [HD][Hd][B][Tp]: Q transposed, each sequence padded with zero rows to Tp
  const void* dOt;   // [HD][Hd][B][Tp]: dO, the same way
  const void* Kt;    // [HD][Hkd][B][Sp]: K transposed, each sequence padded with zero keys to Sp
  const void* Vr;    // [B*S][Hkd*HD]: V by rows
  int64_t T, S, chunk, Tp, Sp;  // Tp, Sp: T and S rounded up to a multiple of 64
  int ldo, ldo_fwd, rank, fold, batch, grp, Hd, Hkd;  // row pitches of dO and O
  float scale_log2, scale;
  int dq_seg, dq_items;  // 64-key blocks per segment; items per (head, sequence)
};
// The dQ kernel's work items: each 128-row query block's keys split into
// segments of at most *seg 64-key blocks, so that the zigzag's long
// second-chunk blocks do not leave half the CUs idle; *items per (head,
// sequence).  heads = query heads x sequences of the launch.
void attn_bwd_dq_plan(int64_t T, int64_t chunk, int rank, int fold, int64_t heads, int* seg, int* items);
// part 0: Dl; 1: dK and dV; 2: dQ (the items, then their merge).
hipError_t launch_attn_bwd(int head_dim, const AttnBwdArgs& a, int part, hipStream_t s);

}  // namespace tsp
