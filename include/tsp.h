/*
 * tsp.h - C ABI of one rank's share of a folded tensor+sequence parallel
 * (TSP) transformer layer, on one AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "Folding Tensor and Sequence Parallelism for
 * Memory-Efficient Transformer Training & Inference" (gist.science summary),
 * section 2 "Metodologia: TSP", main design components.  TSP folds tensor and
 * sequence parallelism onto ONE device axis of D ranks: each rank keeps 1/D
 * of the parameters and 1/D of the tokens.  Attention weight shards are
 * broadcast one per iteration, K/V are all-gathered along the sequence before
 * flash attention, zigzag partitioning balances causal work, and gated-MLP
 * weight shards circulate on a ring while each rank sums its partial outputs
 * locally (no all-reduce).
 *
 * This library computes rank r's share on one GPU.  The other ranks' weight
 * shards and the all-gathered K/V are ordinary device buffers.  The weight
 * shards stream through two workspace slots with copies on a side stream that
 * overlap the compute, in place of the broadcast / ring transfers between
 * GPUs; the other ranks' K/V rows (the all-gather's payload) are read in
 * place by the attention kernel when C is a multiple of 64, and otherwise
 * copied into a slot next to the rank's own rows as well.
 *
 * ---------------------------------------------------------------------------
 * Notation: h hidden, H heads, d = h/H head dim, F FFN width, S sequence
 * length, D fold degree, r rank.  C = S/(2D) zigzag chunk, T = S/D = 2C local
 * tokens, Hd = H/D heads per shard, hs = h/D = Hd*d, Fs = F/D.  Hkv K/V heads
 * (Hkv = H unless dims->n_kv_heads says otherwise), Hkd = Hkv/D K/V heads per
 * shard, ks = Hkd*d, g = H/Hkv query heads per K/V head.
 * b = element size (2 for bf16, 4 for fp32).
 *
 * Layer (pre-norm): x1 = x + Attn(RMSNorm(x; g1)) W_O,
 *                   out = x1 + (silu(n2 W1) * (n2 W3)) W2, n2 = RMSNorm(x1; g2).
 * RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g.  Attention is causal
 * (key position <= query position), scale 1/sqrt(d), no bias.  Query head t
 * reads K/V head t / g (grouped-query attention; g = 1 gives every head its
 * own K/V, the pages' setting).
 *
 * Positional encoding.  The pages name none, and by default there is none.
 * With dims->rope_theta = theta > 0, Q and K carry the rotary position
 * embedding of RoFormer (Su et al., "RoFormer: Enhanced Transformer with
 * Rotary Position Embedding", section 3.2): in every head, the pair of dims
 * (2i, 2i+1) of the row at position p is rotated by the angle
 * p * theta^(-2i/d), i = 0 .. d/2-1, with
 *   out[2i]   = u cos(a) - v sin(a),   out[2i+1] = u sin(a) + v cos(a),
 * (u, v) being the pair before rotation.  p is the token's global position in
 * its sequence, so a rank's zigzag rows carry the angles of the positions
 * they hold, not of their local order.  Angles are reduced modulo 2 pi in
 * double precision before the single-precision sine and cosine.
 *
 * Zigzag layout (section 2, attention layers): the sequence is cut into 2D
 * chunks of C tokens; rank r holds chunk r then chunk 2D-1-r.  Local row
 * i < C is global position r*C + i; local row C + i is (2D-1-r)*C + i.
 *
 * Micro-batch (section 2, results: TSP leaves room for larger micro-batches):
 * B = dims->batch independent sequences of length S share the weights.  Each
 * is zigzag-partitioned as above; local activations are sequence-major,
 * [B*T][h], rows [b*T, (b+1)*T) being sequence b's T local rows, and every
 * query attends only to keys of its own sequence.
 *
 * Weight shards (section 2: attention shards pack W_Q, W_K, W_V, W_O; the MLP
 * shards are W1, W3, W2).  Shard j covers heads [j*Hd, (j+1)*Hd) and FFN
 * columns [j*Fs, (j+1)*Fs).  Every matrix block is stored "output-major"
 * (each row is one output feature, its input features contiguous), so a
 * projection y = a W reads block row n as column n of W:
 *   attention shard j, (2*hs + 2*ks)*h elements, contiguous (4*hs*h when
 *   Hkv = H); W_K and W_V have Hkv*d columns, shard j holding K/V heads
 *   [j*Hkd, (j+1)*Hkd), which serve its query heads:
 *     [0, hs)           rows x h cols : row n = column j*hs + n of W_Q
 *     [hs, hs+ks)       rows x h cols : row n = column j*ks + n of W_K
 *     [hs+ks, hs+2ks)   rows x h cols : row n = column j*ks + n of W_V
 *     then h rows x hs cols           : row n, col k = W_O[j*hs + k][n]
 *   MLP shard j, 3*Fs*h elements, contiguous:
 *     Fs rows x h cols : row n = column j*Fs + n of W1 (gate, through silu)
 *     Fs rows x h cols : row n = column j*Fs + n of W3 (linear branch)
 *     h rows x Fs cols : row n, col k = W2[j*Fs + k][n]
 *
 * Gathered K/V (the all-gather's result), D blocks of 2*Hkd*B*S*d elements;
 * block j = [K_j | Vt_j]:
 *     K_j  [Hkd][B*S][d] : K_j[t][b*S + p][e]  = K of K/V head j*Hkd+t, sequence b, position p, dim e
 *     Vt_j [Hkd][d][B*S] : Vt_j[t][e][b*S + p] = V of K/V head j*Hkd+t, sequence b, position p, dim e
 * V is stored transposed so that the P.V contraction reads keys contiguously.
 * K is stored after the rotary embedding when rope_theta > 0.  With B = 1 and
 * Hkv = H these are [Hd][S][d] and [Hd][d][S].
 *
 * ---------------------------------------------------------------------------
 * Conventions for every entry point
 *   - Device pointers are plain device addresses; host pointer arrays
 *     (w_attn, w_mlp: D entries) are read during the call only.  The caller
 *     owns every buffer; the library allocates no device memory per call.
 *   - All tensors of one call share dims->dtype; accumulation is fp32.
 *     bf16 intermediates: normalised activations, Q/K/V, attention
 *     probabilities, per-shard attention output and the SwiGLU product.
 *   - Device pointers must be 16-byte aligned, tensors contiguous.
 *   - Outputs must not alias inputs or the workspace.
 *   - Streams are hipStream_t passed as void*; NULL means the null stream.
 *     Calls are asynchronous: all work is enqueued on `stream`; side-stream
 *     copies go to `copy_stream` (if NULL or equal to `stream`, copies run
 *     in order on `stream`) and that stream is joined back into `stream`
 *     before the call returns.  No host synchronisation.
 *   - Return 0 (TSP_OK) on success.  Argument errors return a negative code
 *     BEFORE anything is enqueued.  TSP_E_HIP reports a failed launch or
 *     copy; tsp_last_error() gives the detail (thread-local).
 *   - Calls that share a workspace must not overlap in time.
 *   - An empty sequence (S == 0) is valid and enqueues nothing.
 *   - Calls may be captured into a HIP graph (stream capture on `stream`):
 *     everything they enqueue is a kernel, an asynchronous copy or an event
 *     record / wait between `stream` and `copy_stream`, with no host
 *     synchronisation and no memset node.  Make the first call of a host
 *     thread on a device outside capture (it creates the library's events),
 *     and do not capture calls made with TSP_F_PROFILE.
 */
#ifndef TSP_H
#define TSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { TSP_BF16 = 0, TSP_F32 = 1 };

enum {
  TSP_OK = 0,
  TSP_E_INVAL = -1,     /* null pointer, rank outside [0, D), negative size, batch,
                           n_kv_heads or rope_theta */
  TSP_E_SHAPE = -2,     /* h != H*d, H % D, F % D, S % 2D, S % 8, unsupported d,
                           H % Hkv, Hkv % D, or a buffer the kernels stage from
                           would exceed 2^31 bytes: B*T*max(h, G*hs, G*Fs, 2*Fs)*b,
                           G = max(1, min(4, D/2)) (activations, the grouped O / W2 operands, the MLP
                           backward's [da | db]), the weight blocks, or one K/V
                           head's K or V^T plane (the kernels use 32-bit byte
                           offsets within each buffer) */
  TSP_E_ALIGN = -3,     /* a device pointer is not 16-byte aligned */
  TSP_E_WORKSPACE = -4, /* ws_bytes < tsp_workspace_bytes(...) */
  TSP_E_DTYPE = -5,     /* dtype is neither TSP_BF16 nor TSP_F32 */
  TSP_E_HIP = -6        /* a HIP launch or copy failed */
};

/* Workspace kinds for tsp_workspace_bytes. */
enum {
  TSP_WS_ATTN = 1,
  TSP_WS_MLP = 2,
  TSP_WS_LAYER = 3,
  TSP_WS_KV = 4,
  TSP_WS_MLP_BWD = 5,
  TSP_WS_ATTN_BWD = 6,
  TSP_WS_LAYER_BWD = 7,
  TSP_WS_LAYER_BWD_FINISH = 8
};

/* Flags (tsp_dims.flags).  Results must be identical with or without the
 * first four; they exist to expose missing stream hand-offs in tests.
 * TSP_F_RESCALE_TEST changes only the rounding: the bf16 attention with
 * 128-dim heads keeps a lazy softmax reference max and raises it when a
 * 32-key block's exponentials sum past 2^64; with this flag the bound is 2,
 * so the rescale path runs on ordinary inputs. */
enum {
  TSP_F_DELAY_COPY = 1u,   /* a bounded spin kernel runs on the copy stream before each copy */
  TSP_F_POISON_SLOTS = 2u, /* each slot is filled with NaN before it is refilled */
  TSP_F_NO_OVERLAP = 4u,   /* run the copies in order on the compute stream */
  TSP_F_PROFILE = 8u,      /* time each kernel launch with HIP events (tsp_profile_read) */
  TSP_F_RESCALE_TEST = 16u, /* softmax rescale bound 2 instead of 2^64 (see above) */
  /* Route the K/V all-gather's payload through the shard stream at every
   * shape: the other ranks' rows of each head group are copied into a K/V slot
   * on the side stream, overlapped with the previous group's compute, as they
   * are when C % 64 != 0 (section 2, attention layers: the all-gather; section
   * 3: transfers pipelined behind the GEMMs).  Without it they are read in
   * place when C % 64 == 0.  Same results, bit for bit. */
  TSP_F_KV_STREAM = 32u,
  /* Shards per launch and per O / W2 projection.  By default P = max(1,
   * min(4, D/2)) consecutive shards (4 at D = 8, 2 at D = 4) run as one QKV
   * launch and one attention launch once all of them have arrived in a slot,
   * which takes two slots of P shards each; the W1/W3 projection of two such
   * groups runs as one launch over both slots; and one O
   * (W2) projection covers all D shards (K = h, K = F), adding the residual,
   * with all of W_O (W2) copied into one group buffer -- unless the layer's
   * SwiGLU products would exceed 2^31 bytes, when groups of P shards
   * accumulate through an fp32 partial sum.  This flag runs one shard per
   * launch in smaller slots and groups of P shards for the O / W2
   * projections: the stream's smallest footprint.  Results agree to
   * rounding: the attention's work split depends on the heads per launch,
   * the projections' sums on the grouping. */
  TSP_F_SHARD_LAUNCH = 64u
};

/* Kernel classes reported by tsp_profile_read. */
enum {
  TSP_K_RMSNORM = 0, /* RMSNorm of the rank's tokens */
  TSP_K_QKV = 1,     /* QKV projection of a launch's attention shards (+ K/V scatter) */
  TSP_K_ATTN = 2,    /* zigzag causal flash attention of a launch's head groups */
  TSP_K_MERGE = 3,   /* merge of split attention work items */
  TSP_K_OPROJ = 4,   /* O projection of a group of shards (all of them by default), + residual */
  TSP_K_W13 = 5,     /* W1/W3 projection of a launch's MLP shards with the SwiGLU product */
  TSP_K_W2 = 6,      /* W2 projection of a group of shards (all of them by default), + residual */
  TSP_K_COUNT = 7
};

typedef struct tsp_dims {
  int32_t hidden;   /* h */
  int32_t n_heads;  /* H */
  int32_t head_dim; /* d; supported: 16, 32, 64, 128 */
  int32_t ffn;      /* F */
  int32_t fold;     /* D, ranks on the TSP axis */
  int32_t rank;     /* r in [0, D) */
  int64_t seq;      /* S, total sequence length */
  float eps;        /* RMSNorm epsilon (inside the square root) */
  int32_t dtype;    /* TSP_BF16 or TSP_F32 */
  uint32_t flags;   /* TSP_F_* */
  int32_t batch;    /* B, micro-batch of independent sequences (0 means 1) */
  int32_t n_kv_heads; /* Hkv, K/V heads; 0 means H.  H % Hkv == 0, Hkv % D == 0 */
  float rope_theta;   /* rotary embedding base theta; 0 means no rotary embedding */
} tsp_dims;

/* Bytes of workspace an entry point needs for these dims (0 on bad dims). */
size_t tsp_workspace_bytes(const tsp_dims* dims, int which);

/* Static description of a status code. */
const char* tsp_strerror(int status);

/* Detail of the last error returned on this host thread ("" if none). */
const char* tsp_last_error(void);

/* Host helper: writes the T = S/D global positions of rank r's local rows
 * (zigzag layout above) into out[0..T).  Returns TSP_E_SHAPE if S % 2D. */
int tsp_zigzag_positions(int64_t seq, int32_t fold, int32_t rank, int64_t* out);

/*
 * Attention half of rank r's layer share: x1 = x + Attn(RMSNorm(x; g1)) W_O.
 * Section 2, attention layers: for broadcast iteration j = 0..D-1 the packed
 * shard j is used (w_attn[r] is read in place, the others are copied into a
 * workspace slot on the side stream), the rank projects its own tokens to
 * Q_j/K_j/V_j, zigzag-aware causal flash attention runs over the gathered
 * K/V (the rank's own rows from the projection, the other ranks' rows its
 * causal window needs, positions < (2D-r)*C, from `kv`: read in place when
 * C % 64 == 0, else -- or always with TSP_F_KV_STREAM -- first copied next to
 * its own on the side stream), and the partial
 * O-projection of head group j is accumulated locally in fp32.
 *   x      [B*T][h] local rows in zigzag order, sequence-major
 *   g1     [h]      RMSNorm gain
 *   w_attn D device pointers to packed attention shards (layout above)
 *   kv     gathered K/V (layout above); only other ranks' rows are read
 *   x1     [B*T][h] output
 *   ws     workspace of at least tsp_workspace_bytes(dims, TSP_WS_ATTN) bytes
 */
int tsp_attn_shard(const tsp_dims* dims, const void* x, const void* g1,
                   const void* const* w_attn, const void* kv, void* x1,
                   void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/*
 * tsp_attn_shard for training: the same x1 (bit for bit), and it also keeps
 * what the backward would otherwise recompute (FlashAttention's backward
 * takes the forward output and the softmax statistics as inputs):
 *   attn_out [B*T][h] dims->dtype: every head group's attention output, the
 *            input of its O projection (shard j's heads at columns j*hs)
 *   lse      [H][B*T] fp32: log2 of each row's softmax normaliser over the
 *            scaled scores (head t = j*Hd + u of shard j at row block t)
 * Both are overwritten; pass them to tsp_layer_shard_backward.
 *   ws >= tsp_workspace_bytes(dims, TSP_WS_ATTN).
 */
int tsp_attn_shard_save(const tsp_dims* dims, const void* x, const void* g1,
                        const void* const* w_attn, const void* kv, void* x1,
                        void* attn_out, float* lse, void* ws, size_t ws_bytes,
                        void* stream, void* copy_stream);

/*
 * MLP half: out = x1 + sum_j (silu(n2 W1_j) * (n2 W3_j)) W2_j, n2 = RMSNorm(x1; g2).
 * Section 2, gated MLP layers: ring step t = 0..D-1 uses shard (r + t) mod D
 * (own shard first, read in place; the others are copied into a workspace
 * slot on the side stream); the partial outputs are summed locally in fp32,
 * so no all-reduce is needed.
 *   x1    [B*T][h], g2 [h], w_mlp D device pointers to packed MLP shards,
 *   out   [B*T][h], ws >= tsp_workspace_bytes(dims, TSP_WS_MLP).
 */
int tsp_mlp_shard(const tsp_dims* dims, const void* x1, const void* g2,
                  const void* const* w_mlp, void* out,
                  void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/*
 * Whole layer share: tsp_attn_shard then tsp_mlp_shard, with x1 kept in the
 * workspace and the first MLP shard copies issued while attention runs.
 *   ws >= tsp_workspace_bytes(dims, TSP_WS_LAYER).
 */
int tsp_layer_shard(const tsp_dims* dims, const void* x, const void* g1,
                    const void* const* w_attn, const void* kv, const void* g2,
                    const void* const* w_mlp, void* out,
                    void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/*
 * tsp_layer_shard without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results (bit for bit) as tsp_layer_shard; the
 * workspace is instead a static device array of TSP_NOALLOC_SCRATCH_BYTES
 * (256 MiB: the 7B-shape layer share fits up to S = 4096 at D = 8 with
 * TSP_F_SHARD_LAUNCH) that the
 * library holds on every GPU it runs on until the process ends.
 *   - Returns TSP_E_WORKSPACE, before anything is enqueued, when the dims
 *     need more than that (tsp_workspace_bytes(dims, TSP_WS_LAYER) tells).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on the same GPU (other streams, other host threads) race and
 *     must not be made.  The array keeps the last call's contents; no result
 *     depends on them.
 *   - It calls no hipMalloc, hipFree or allocating library routine.  The
 *     first call on a device looks up the array's device address once; as
 *     with every entry point, the first call of a host thread on a device
 *     creates that thread's HIP events.  TSP_F_PROFILE is refused
 *     (TSP_E_INVAL): it creates timing events per launch.
 */
#define TSP_NOALLOC_SCRATCH_BYTES (256ull << 20)
int tsp_layer_shard_noalloc(const tsp_dims* dims, const void* x, const void* g1,
                            const void* const* w_attn, const void* kv, const void* g2,
                            const void* const* w_mlp, void* out, void* stream, void* copy_stream);

/*
 * Rank r's contribution to the K/V all-gather (section 2, attention layers:
 * the all-gather rebuilds full-length K/V along the sequence): writes K and
 * V of rank r's local tokens, for every head, at their global positions into
 * `kv` (layout above).  Rows of other ranks are left untouched.
 *   x [B*T][h], g1 [h], w_attn D device pointers, ws >= tsp_workspace_bytes(dims, TSP_WS_KV).
 */
int tsp_kv_shard(const tsp_dims* dims, const void* x, const void* g1,
                 const void* const* w_attn, void* kv,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the MLP half for rank r's rows (training; the pages describe
 * only the forward schedules, so this follows the plainest reading of them:
 * the gradient of the rank's own rows goes through the MLP locally, and each
 * weight shard gets a PARTIAL gradient from these rows, which a
 * reduce-scatter over the D ranks would sum at the shard's owner, the reverse
 * of the ring).  With n2 = RMSNorm(x1; g2), a_j = n2 W1_j, b_j = n2 W3_j,
 * out = x1 + sum_j (silu(a_j) * b_j) W2_j and the output gradient dout:
 *   x1     [B*T][h]  the forward input of the MLP half
 *   g2     [h]       RMSNorm gain
 *   w_mlp  D device pointers to packed MLP shards (as tsp_mlp_shard)
 *   dout   [B*T][h]  gradient of out
 *   dx1    [B*T][h]  output: gradient of x1 (dout through the residual plus the
 *                    MLP branch through the norm), in dims->dtype
 *   dg2    [h] fp32  output: this rank's partial gradient of g2 (overwritten)
 *   dw_mlp D device pointers, each 3*Fs*h fp32 elements: output, this rank's
 *          partial gradient of shard j in the shard's packed layout (dW1 rows,
 *          dW3 rows, then the dW2 block), overwritten
 *   ws     workspace of at least tsp_workspace_bytes(dims, TSP_WS_MLP_BWD) bytes
 * Everything is enqueued on `stream` (no side stream); products accumulate in
 * fp32, [da | db] and g = silu(a) b are stored in dims->dtype as GEMM operands.
 */
int tsp_mlp_shard_backward(const tsp_dims* dims, const void* x1, const void* g2,
                           const void* const* w_mlp, const void* dout, void* dx1, float* dg2,
                           float* const* dw_mlp, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the causal attention core for one shard's head group (Hd = H/D
 * query heads, Hkd = Hkv/D K/V heads) over rank r's rows, training as above.
 * The gradient is that of o = softmax(q k^T / sqrt(d), keys at or before the
 * query's global zigzag position) v ("Folding Tensor and Sequence
 * Parallelism ...", section 2: each rank's queries attend to the gathered
 * full-length K/V), computed as FlashAttention does: the forward's per-row
 * log-sum-exp is recomputed from q and kv, then the probabilities are rebuilt
 * block by block, so nothing of size S x S is stored.
 *   q     [Hd][B*T][d]      the group's rotated queries (the QKV step's layout)
 *   kv    K [Hkd][B*S][d], then V^T [Hkd][d][B*S]: every position's keys
 *         (rotated) and values, as tsp_attn_shard reads them
 *   dout  [B*T][Hd*d]       gradient of the group's attention output, head t
 *                           at columns [t*d, (t+1)*d)
 *   dq    [Hd][B*T][d] fp32 output: gradient of q (overwritten)
 *   dk    [Hkd][B*S][d] fp32 output: this rank's PARTIAL gradient of every
 *                           position's key, zero where no query of the rank
 *                           attends (a reduce-scatter over the ranks, the
 *                           reverse of the K/V all-gather, would sum them at
 *                           each position's owner)
 *   dv    [Hkd][B*S][d] fp32 output: the same for the values
 *   ws    workspace of at least tsp_workspace_bytes(dims, TSP_WS_ATTN_BWD) bytes
 * bf16 only (TSP_E_DTYPE otherwise), head_dim 64 or 128 (TSP_E_SHAPE
 * otherwise).  Products accumulate in fp32; the probabilities and dS enter
 * the MFMA products in bf16.  Everything is enqueued on `stream`.
 */
int tsp_attn_core_backward(const tsp_dims* dims, const void* q, const void* kv, const void* dout,
                           float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of rank r's whole layer share (training), in two parts around the
 * one exchange the gradient needs.  The pages give the forward schedules
 * only ("Folding Tensor and Sequence Parallelism ...", section 2: attention
 * shards broadcast, K/V all-gathered along the sequence, MLP shards on a
 * ring, partial outputs summed locally); the backward follows the plainest
 * reading of them: the rank takes the gradient of its own zigzag rows
 * through the layer, forms a PARTIAL gradient of every weight shard from
 * those rows (a reduce-scatter over the D ranks, the reverse of the
 * broadcast and the ring, sums the partials at each shard's owner), and its
 * queries produce gradients for the K/V of every position they attended to,
 * which a reduce-scatter (the reverse of the K/V all-gather) sums at the
 * positions' owners before the owners take them through W_K, W_V and the
 * norm.  bf16 only with head_dim 64 or 128 (TSP_E_DTYPE / TSP_E_SHAPE
 * otherwise), as the attention core's backward.  Everything is enqueued on
 * `stream`; weight shards are read in place.
 *
 * Part 1, before the exchange.  With the forward's inputs and its
 * attention-half output x1 (which training keeps), and the output gradient:
 *   x, x1   [B*T][h]   the layer's input and tsp_attn_shard's output
 *   g1, w_attn, kv, g2, w_mlp   as the forward (kv: the gathered K/V; every
 *           other rank's rows are read, the rank's own are recomputed)
 *   dout    [B*T][h]   gradient of the layer output
 *   attn_saved, lse_saved   the attn_out and lse of tsp_attn_shard_save on
 *           the same inputs, or both NULL (TSP_E_INVAL if only one is given)
 * outputs (all overwritten):
 *   dx1     [B*T][h]   gradient of x1 (dout plus the MLP branch), dims->dtype
 *   dg2     [h] fp32   partial gradient of g2
 *   dw_mlp  D pointers, 3*Fs*h fp32 each: partial gradients of the MLP
 *           shards in their packed layout (as tsp_mlp_shard_backward)
 *   dw_o    D pointers, h*hs fp32 each: partial gradient of each shard's W_O
 *           block in its packed layout (row n, column k: dW_O[j*hs + k][n])
 *   dq      [H][B*T][d] fp32: gradient of the rank's queries before the
 *           rotation (head t = j*Hd + u of shard j at block t)
 *   dkv     D blocks of [2][Hkd][B*S][d] fp32 (block j: dK then dV of K/V
 *           heads [j*Hkd, (j+1)*Hkd), every position of every sequence,
 *           keys before the rotation): this rank's partial K/V gradients,
 *           zero at positions none of its queries sees
 *   ws      >= tsp_workspace_bytes(dims, TSP_WS_LAYER_BWD)
 * Without attn_saved / lse_saved, the forward attention of each head group
 * is recomputed (FlashAttention's way); RMSNorm-1, Q and the rank's own K/V
 * rows are recomputed either way.
 */
int tsp_layer_shard_backward(const tsp_dims* dims, const void* x, const void* x1, const void* g1,
                             const void* const* w_attn, const void* kv, const void* g2,
                             const void* const* w_mlp, const void* dout, const void* attn_saved,
                             const float* lse_saved, void* dx1, float* dg2,
                             float* const* dw_mlp, float* const* dw_o, float* dq, float* dkv,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * The exchange's arithmetic for rank r (a harness helper, like tsp_kv_shard:
 * on D GPUs a reduce-scatter does this): dkv_own = the sum over the D ranks'
 * part-1 dkv buffers, taken at rank r's positions,
 *   dkv_own[j][c][t][b*T + i][e] = sum_q dkv_parts[q][j][c][t][b*S + zig_r(i)][e],
 * a [D][2][Hkd][B*T][d] fp32 buffer (c: K or V).  dkv_parts: D device
 * pointers (host array).  TSP_E_SHAPE if D > 64.
 */
int tsp_kv_grad_reduce(const tsp_dims* dims, const float* const* dkv_parts, float* dkv_own, void* stream);

/*
 * Part 2, after the exchange: the rank's own rows through W_Q, W_K, W_V and
 * RMSNorm-1.  With dq from part 1 and dkv_own from tsp_kv_grad_reduce:
 *   dn1 = sum_j [dQ_j | dK_j | dV_j] [W_Q_j; W_K_j; W_V_j]^T
 *   dx  [B*T][h]  = dx1 + RMSNorm-1's backward of dn1, dims->dtype
 *   dg1 [h] fp32  partial gradient of g1 (overwritten)
 *   dw_qkv D pointers, (hs + 2*ks)*h fp32 each: partial gradient of each
 *          shard's Q|K|V block in its packed layout (row n, column k: the
 *          gradient of that block's element), overwritten
 *   ws  >= tsp_workspace_bytes(dims, TSP_WS_LAYER_BWD_FINISH)
 * The W_O rows of a packed shard are not touched (part 1 gives dw_o).
 */
int tsp_layer_shard_backward_finish(const tsp_dims* dims, const void* x, const void* g1,
                                    const void* const* w_attn, const void* dx1, const float* dq,
                                    const float* dkv_own, void* dx, float* dg1, float* const* dw_qkv,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * Per-kernel timing of calls made with TSP_F_PROFILE: every kernel the
 * library launches on the compute stream is bracketed by two HIP events on
 * that stream.  tsp_profile_read waits for the recorded events, adds their
 * elapsed times into per-class totals and writes, for each class k in
 * [0, TSP_K_COUNT), the total milliseconds ms[k] and the launch count n[k]
 * since the last reset (either pointer may be NULL).  reset != 0 clears the
 * totals afterwards.  State is per host thread; events of one thread must
 * all belong to the device current at the read.  The timing events cost a
 * few microseconds per launch, so calls timed this way are slightly slower.
 */
int tsp_profile_read(double* ms, int64_t* n, int reset);

/*
 * Effective graphics clock, for measurement: enqueues on `stream` a one-wave
 * kernel that writes n pairs (wall-clock tick, shader-clock cycle) into the
 * device buffer samples[2n], one every interval_us microseconds, and writes
 * the wall clock's rate (kHz) to *wall_khz.  The shader clock counts at the
 * clock the chip sustains (under its power limit it runs below the
 * configured one); so, launched on a second stream beside other work, the
 * probe reads the clock that work ran at: f = delta(cycles) / delta(ticks) *
 * wall_khz.  The probe occupies one wave slot of one CU and sleeps between
 * samples.  TSP_E_INVAL if n <= 0, interval_us <= 0 or n * interval_us
 * exceeds 4 s; TSP_E_ALIGN if samples is not 8-byte aligned.
 */
int tsp_clock_probe(uint64_t* samples, int32_t n, int32_t interval_us, int32_t* wall_khz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSP_H */
