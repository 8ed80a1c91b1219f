// gfx950 kernels of one TSP rank's layer share: RMSNorm, the projection GEMM
// (bf16 / fp32 MFMA, fused epilogues) and zigzag-aware causal flash attention.
//
// Method: "Folding Tensor and Sequence Parallelism for Memory-Efficient
// Transformer Training & Inference", section 2 (local projections of the
// rank's own tokens with each weight shard, flash attention of the local
// queries against the all-gathered K/V, zigzag partitioning, local
// accumulation of partial outputs).  The attention kernel follows the
// published FlashAttention method (tiles of K/V streamed through on-chip
// memory, running max and running sum of the softmax, one rescale per tile).
//
// MFMA conventions relied on (32x32 output block, v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2_f32): lane l supplies row l%32 of A and column l%32 of B,
// lanes 0-31 and 32-63 cover the two halves of the k range with the same
// assignment for A and B; the result element (row, col) lives in lane
// col + 32*((row/4)%2), register 4*(row/8) + row%4.
#include "tsp_kernels.h"

#include <math.h>

#include <algorithm>
#include <type_traits>
#include <vector>

namespace tsp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct MF;
template <>
struct MF<bf16> {
  static constexpr int KSTEP = 16;  // k per instruction
  static constexpr int E = 8;       // operand elements per lane
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MF<float> {
  static constexpr int KSTEP = 2;
  static constexpr int E = 1;
  typedef float frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ inline float to_f(bf16 v) { return (float)v; }
__device__ inline float to_f(float v) { return v; }
template <typename T>
__device__ inline T from_f(float v);
template <>
__device__ inline bf16 from_f<bf16>(float v) { return (bf16)v; }
template <>
__device__ inline float from_f<float>(float v) { return v; }

template <typename T>
union Chunk {  // one 16-byte vector
  u32x4 raw;
  T e[16 / sizeof(T)];
};

// Zigzag layout: local row i < C is global position r*C + i, row C + i is
// (2D-1-r)*C + i (section 2, attention layers: zigzag partitioning).
__device__ __host__ inline int64_t zig(int64_t row, int64_t C, int rank, int fold) {
  return row < C ? rank * C + row : (int64_t)(2 * fold - 1 - rank) * C + (row - C);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotary position embedding (RoFormer, section 3.2) of four consecutive head
// dims e..e+3 (e even): pair (2i, 2i+1) turns by p * theta^(-2i/d).  The angle
// is formed and reduced modulo 2 pi in double precision (at p ~ 1e5 a
// single-precision product would be off by ~1e-2 rad); sine and cosine of the
// reduced angle are single precision.
// l2c = log2(theta) / d.
__device__ inline void rope_pairs(float* v, int e, int64_t p, double l2c) {
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int i = e / 2 + t;
    const double ang = (double)p * exp2(-(double)(2 * i) * l2c);
    const double k = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
    const float red = (float)fma(-k, 6.283185307179586, ang);
    float sn, cs;
    sincosf(red, &sn, &cs);
    const float u = v[2 * t], w = v[2 * t + 1];
    v[2 * t] = u * cs - w * sn;
    v[2 * t + 1] = u * sn + w * cs;
  }
}

// ---------------------------------------------------------------------------
// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, fp32 math, one wave per row.
// HBM-bound.  Rows of up to 64*RC 16-byte chunks (8192 bf16, 4096 fp32) are
// read once into registers, all loads in flight together, and scaled from
// there; wider or unaligned rows are read a second time for the scaled write.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const T* __restrict__ x,
                                                      const T* __restrict__ g,
                                                      T* __restrict__ y, int64_t rows, int h,
                                                      float eps) {
  constexpr int V = 16 / sizeof(T);
  constexpr int RC = 16;  // 16-byte chunks per lane held in registers
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + row * h;
  T* yr = y + row * h;
  const bool vec = (h % V) == 0;
  float ss = 0.f;
  if (vec && h / V <= 64 * RC) {
    const int nc = h / V;
    Chunk<T> v[RC];
#pragma unroll
    for (int k = 0; k < RC; k++) {
      const int c = lane + 64 * k;
      v[k].raw = c < nc ? *(const u32x4*)(xr + (int64_t)c * V) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < RC; k++)
#pragma unroll
      for (int i = 0; i < V; i++) {
        const float f = to_f(v[k].e[i]);
        ss += f * f;
      }
#pragma unroll
    for (int o = 32; o; o >>= 1) ss += __shfl_xor(ss, o);
    const float rs = 1.0f / sqrtf(ss / (float)h + eps);
#pragma unroll
    for (int k = 0; k < RC; k++) {
      const int c = lane + 64 * k;
      if (c < nc) {
        Chunk<T> w, out;
        w.raw = *(const u32x4*)(g + (int64_t)c * V);
#pragma unroll
        for (int i = 0; i < V; i++) out.e[i] = from_f<T>(to_f(v[k].e[i]) * rs * to_f(w.e[i]));
        *(u32x4*)(yr + (int64_t)c * V) = out.raw;
      }
    }
    return;
  }
  if (vec) {
    for (int c = lane; c < h / V; c += 64) {
      Chunk<T> v;
      v.raw = *(const u32x4*)(xr + (int64_t)c * V);
#pragma unroll
      for (int i = 0; i < V; i++) {
        const float f = to_f(v.e[i]);
        ss += f * f;
      }
    }
  } else {
    for (int i = lane; i < h; i += 64) {
      const float f = to_f(xr[i]);
      ss += f * f;
    }
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) ss += __shfl_xor(ss, o);
  const float rs = 1.0f / sqrtf(ss / (float)h + eps);
  if (vec) {
    for (int c = lane; c < h / V; c += 64) {
      Chunk<T> v, w, out;
      v.raw = *(const u32x4*)(xr + (int64_t)c * V);
      w.raw = *(const u32x4*)(g + (int64_t)c * V);
#pragma unroll
      for (int i = 0; i < V; i++) out.e[i] = from_f<T>(to_f(v.e[i]) * rs * to_f(w.e[i]));
      *(u32x4*)(yr + (int64_t)c * V) = out.raw;
    }
  } else {
    for (int i = lane; i < h; i += 64) yr[i] = from_f<T>(to_f(xr[i]) * rs * to_f(g[i]));
  }
}

// ---------------------------------------------------------------------------
// Projection GEMM: acc = A . B^T, A [M][K] (lda), B [N][K] (ldb), both
// K-contiguous.  256 threads = 2x2 waves; each wave owns (BM/2) x (BN/2) of
// the tile as 32x32 MFMA blocks.  K is staged through LDS in 128-byte rows
// (64 bf16 / 32 fp32), double-buffered.  LDS rows are XOR-swizzled in
// 16-byte chunks so the 32 rows one fragment read touches spread over the
// banks.
//
// Vector path (K, lda, ldb multiples of 16 bytes): tiles go straight from
// global memory to LDS with buffer loads (no staging registers); rows past M
// or N and chunks past K read as zero through the buffer's range check.  One
// barrier per K step: after it every wave's loads of this step have landed
// and every wave has finished reading the other buffer, which the next
// step's loads then refill while this step's MFMAs run.  Scalar path (odd
// sizes): element-wise guarded loads through registers.
//
// The MFMA takes B's fragment as its first operand, so a lane of the 32x32
// result holds one output row m and, per group of four registers, four
// consecutive columns n: the epilogues use 4-wide loads and stores.
// ---------------------------------------------------------------------------
// XOR swizzle of the 16-byte chunk c in row r of an LDS tile with NCH chunks
// per row.  The LDS has 64 banks of 4 bytes (256 bytes per sweep) and serves
// a 16-byte read for 16 lanes at a time, so 16 consecutive rows read at one
// logical chunk must land on 16 different 16-byte bank groups: the rows that
// share a sweep position (r / (16 / NCH) for rows shorter than a sweep) get
// different XOR terms.
template <int NCH>
__device__ __host__ inline int swz(int c, int r) {
  if constexpr (NCH >= 16)
    return c ^ (r & 15);
  else
    return c ^ ((r / (16 / NCH)) & (NCH - 1));
}

template <typename T, bool VEC>
__device__ inline u32x4 load_chunk(const T* base, bool rowok, int64_t row, int64_t ld, int k,
                                   int K) {
  constexpr int V = 16 / sizeof(T);
  Chunk<T> r;
  r.raw = u32x4{0u, 0u, 0u, 0u};
  if (!rowok) return r.raw;
  const T* p = base + row * ld + k;
  if (VEC) {
    if (k < K) r.raw = *(const u32x4*)p;
  } else {
#pragma unroll
    for (int e = 0; e < V; e++) r.e[e] = (k + e < K) ? p[e] : from_f<T>(0.f);
  }
  return r.raw;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Buffer resources and buffer->LDS loads exist only in the device pass; the
// host pass (which emits the launch stubs) sees inert placeholders.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t brsrc;
#else
typedef const void* brsrc;
#endif

__device__ inline brsrc make_rsrc(const void* p, uint64_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)n, 0x00020000);
#else
  return p;
#endif
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16*lane
// (lds must be the same for every lane of the wave).
__device__ inline void buffer_to_lds16(brsrc r, void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
#endif
}

constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past any range: reads 0

// Max and sum of a value with the lane 32 positions away, through the
// cross-half lane swap (no LDS round trip): after the swap the two results
// hold the lane's own value and its partner's, in an order that depends on
// the half, so their max or sum is the same in both halves.
__device__ inline float halves_max(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
  return x;
#endif
}
__device__ inline float halves_sum(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
#else
  return x;
#endif
}

template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    Chunk<T> v;
    v.e[0] = from_f<T>(a);
    v.e[1] = from_f<T>(b);
    v.e[2] = from_f<T>(c);
    v.e[3] = from_f<T>(d);
    *(u32x2*)p = u32x2{v.raw[0], v.raw[1]};
  } else {
    *(float4*)p = make_float4(a, b, c, d);
  }
}

template <typename T>
__device__ inline void load4(const T* p, float* o) {
  if constexpr (sizeof(T) == 2) {
    Chunk<T> v;
    const u32x2 r = *(const u32x2*)p;
    v.raw[0] = r[0];
    v.raw[1] = r[1];
#pragma unroll
    for (int t = 0; t < 4; t++) o[t] = to_f(v.e[t]);
  } else {
    const float4 r = *(const float4*)p;
    o[0] = r.x;
    o[1] = r.y;
    o[2] = r.z;
    o[3] = r.w;
  }
}

#ifndef TSP_GEMM_GROUP
#define TSP_GEMM_GROUP 0   // grouped tile order for every GEMM, not only QKV (gemm_kernel)
#endif
template <typename T, int BM, int BN, int EPI, bool VEC, int NW, int WGM>
__global__ void __launch_bounds__(NW * 64) gemm_kernel(GemmArgs g) {
  typedef MF<T> M_;
  typedef typename M_::frag frag;
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr bool QKVE = EPI == EPI_QKV || EPI == EPI_QKV_ROPE;  // the Q/K/V scatter epilogue
  constexpr bool ROPE = EPI == EPI_QKV_ROPE;                    // ... with the rotary embedding
  constexpr int ES = sizeof(T);
  constexpr int V = 16 / ES;
  constexpr int BK = 128 / ES;  // elements per 128-byte LDS row
  constexpr int KS = BK / M_::KSTEP;
  constexpr int NT = NW * 64;              // threads
  constexpr int WGN = NW / WGM;            // waves along N (WGM along M)
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int NBR = DUAL ? 2 * BN : BN;  // B rows staged per tile
  constexpr int AC = BM * 8 / NT;          // 16-byte chunks per thread
  constexpr int BC = NBR * 8 / NT;
  constexpr int RR = NT / 8;               // tile rows one load round covers
  constexpr int STAGE = (BM + NBR) * 128;
  constexpr int NB3 = DUAL ? NB : 1;
  static_assert(BM % 64 == 0 && BN % 64 == 0 || BN == 192 || BN == 96, "tile");
  // Ping-pong schedule (below): 8 waves, 16-bit operands, and the split A
  // buffers plus the three-slot B ring must fit in LDS.  Used for the
  // 256x256 single-B tiles, where it measured faster than the lockstep loop
  // (on 256x192 it did not).
  constexpr int PPLDS = 2 * BM * 128 + 3 * NBR * 128;
  constexpr bool PP = VEC && NW == 8 && sizeof(T) == 2 && PPLDS <= 160 * 1024 &&
                      (NBR / 32) % 2 == 0 && BM == 256 && BN == 256 && !DUAL;
  __shared__ __attribute__((aligned(16))) char smem[PP ? PPLDS : 2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lr = lane & 31, lg = lane >> 5;
  const int wm = wave / WGN, wn = wave % WGN;

  // Tiles are handed out so that each XCD (workgroups b with equal b % 8)
  // works on a contiguous range of tiles and shares operands in its L2.
  const int ntn = (g.N + BN - 1) / BN;
  const int nt = gridDim.x;
  const int bid = blockIdx.x;
  const int per = nt >> 3;
  const int t = bid < per * 8 ? (bid & 7) * per + (bid >> 3) : bid;
  // For the QKV and W1/W3 projections (and every GEMM under TSP_GEMM_GROUP)
  // the tiles of that range go in groups of GM tile rows, column by column
  // inside a group, so the tiles an XCD has in flight (32 of 8 waves, 64 of
  // 4 waves) form a GM x 8 block: per k-step they read GM A slices and 8 B
  // slices instead of two full tile rows' worth of B.  Measured in the layer
  // with two shards per launch: W1/W3 1% faster at the 64K workload and 9% at
  // 16K, QKV 4% faster at 64K; the O projection 3% slower, so the
  // accumulating GEMMs keep row order.
  constexpr bool GROUPED = TSP_GEMM_GROUP != 0 || QKVE || EPI == EPI_SWIGLU;
  int m0, n0;
  if constexpr (GROUPED) {
    constexpr int GM = NW == 8 ? 4 : 8;
    const int ntm = (g.M + BM - 1) / BM;
    const int gsz = GM * ntn, grp = t / gsz, first = grp * GM;
    const int rows = min(GM, ntm - first), li = t - grp * gsz;
    m0 = (first + li % rows) * BM;
    n0 = (li / rows) * BN;
  } else {
    m0 = (t / ntn) * BM;
    n0 = (t % ntn) * BN;
  }

  const T* A = (const T*)g.A;
  const T* B = (const T*)g.B;
  const T* B3 = (const T*)g.B3;
  // B rows of this tile's columns: n0 - nb (W1/W3 over two weight blocks; the
  // launcher puts the split on a tile boundary), out of nbr rows
  int nb = 0, nbr = g.N;
  if (DUAL && g.n_split > 0) {
    if (n0 >= g.n_split) {
      B = (const T*)g.B_2;
      B3 = (const T*)g.B3_2;
      nb = g.n_split;
      nbr = g.N - g.n_split;
    } else {
      nbr = g.n_split;
    }
  }
  const int nk = (g.K + BK - 1) / BK;

  f32x16 acc[MB][NB];
  f32x16 acc3[DUAL ? MB : 1][NB3];
#pragma unroll
  for (int i = 0; i < MB; i++)
#pragma unroll
    for (int j = 0; j < NB; j++) {
      acc[i][j] = f32x16{0};
      if (DUAL) acc3[i][j] = f32x16{0};
    }

  frag af[2][MB], bfr[2][NB], bf3[2][NB3];
  // Fragment reads of k-step ks of LDS buffer buf into register set `set`.
  auto fetch = [&](int buf, int ks, int set) {
    const char* sA = smem + buf * STAGE;
    const char* sB = sA + BM * 128;
    const int byte = (ks * M_::KSTEP + lg * M_::E) * ES;
    const int c = byte >> 4, w = byte & 15;
#pragma unroll
    for (int i = 0; i < MB; i++) {
      const int row = wm * WM + i * 32 + lr;
      af[set][i] = *(const frag*)(sA + row * 128 + (swz<8>(c, row) << 4) + w);
    }
#pragma unroll
    for (int j = 0; j < NB; j++) {
      const int row = wn * WN + j * 32 + lr;
      bfr[set][j] = *(const frag*)(sB + row * 128 + (swz<8>(c, row) << 4) + w);
      if (DUAL) {
        const int r3 = BN + row;
        bf3[set][j] = *(const frag*)(sB + r3 * 128 + (swz<8>(c, r3) << 4) + w);
      }
    }
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
      for (int j = 0; j < NB; j++) {
        acc[i][j] = M_::mma(bfr[set][j], af[set][i], acc[i][j]);
        if (DUAL) acc3[i][j] = M_::mma(bf3[set][j], af[set][i], acc3[i][j]);
      }
  };
  // Interleave the fragment reads of the next k-step with this k-step's
  // MFMAs: each read after a group of MFMAs.
  auto interleave = [&]() {
    constexpr int NR = MB + NB + NB3 * (DUAL ? 1 : 0);
    constexpr int NM = MB * NB * (DUAL ? 2 : 1);
    constexpr int PER = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
    for (int q = 0; q < NR; q++) {
      __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // then one DS read
    }
  };
  // k-steps 0 .. KS-2 of buffer buf (fragments of step 0 already in set 0).
  auto compute_head = [&](int buf) {
    __builtin_amdgcn_s_setprio(1);  // wave priority up around the MFMA-heavy k-steps
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ks++) {
      fetch(buf, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
      interleave();
    }
    __builtin_amdgcn_s_setprio(0);
  };
  constexpr int LAST = (KS - 1) & 1;  // register set of the last k-step

  if constexpr (VEC) {
    // Direct global -> LDS.  Load round i of A covers tile rows [RR*i, RR*i+RR);
    // wave w writes rows RR*i + 8w .. +8 (1 KB), lane l the 16 bytes at
    // physical chunk l%8 of row RR*i + 8w + l/8, i.e. logical chunk
    // (l%8) ^ (row%8).
    const brsrc rA = make_rsrc(A, (uint64_t)g.M * g.lda * ES);
    const brsrc rB = make_rsrc(B, (uint64_t)nbr * g.ldb * ES);
    const brsrc rB3 = make_rsrc(DUAL ? B3 : B, (uint64_t)nbr * g.ldb * ES);
    const int lrow = 8 * wave + (lane >> 3);
    // logical chunk of this lane's physical chunk lane%8 (round offsets RR*i
    // are multiples of 16 rows, so the swizzle term depends on lrow only)
    const int lc = swz<8>(lane & 7, lrow);
    uint32_t offA[AC], offB[BC];
#pragma unroll
    for (int i = 0; i < AC; i++) {
      const int gm = m0 + RR * i + lrow;
      offA[i] = gm < g.M ? (uint32_t)(((int64_t)gm * g.lda + lc * V) * ES) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < BC; i++) {
      const int rr = RR * i + lrow;
      const int gn = n0 - nb + (DUAL && rr >= BN ? rr - BN : rr);
      offB[i] = gn < nbr ? (uint32_t)(((int64_t)gn * g.ldb + lc * V) * ES) : kOOB;
    }
    auto issue = [&](int kt, int buf) {
      const int k0 = kt * BK;
      const bool kok = k0 + lc * V < g.K;
      char* sA = smem + buf * STAGE;
      char* sB = sA + BM * 128;
#pragma unroll
      for (int i = 0; i < AC; i++)
        buffer_to_lds16(rA, sA + i * RR * 128 + wave * 1024, kok ? offA[i] : kOOB, k0 * ES);
#pragma unroll
      for (int i = 0; i < BC; i++) {
        const bool second = DUAL && RR * i >= BN;
        buffer_to_lds16(second ? rB3 : rB, sB + i * RR * 128 + wave * 1024, kok ? offB[i] : kOOB,
                        k0 * ES);
      }
    };
    if constexpr (PP) {
      // Ping-pong schedule.  SIMD s runs waves s (group 0) and s + 4 (group
      // 1).  Time is cut into phases separated by workgroup barriers; in
      // each phase one group only issues MFMAs on fragments already in
      // registers while the other only moves data: its fragment reads of the
      // next k-tile and its half of the global->LDS loads.  Group 1 runs one
      // phase behind group 0, so each SIMD has one wave feeding the matrix
      // core while the other waits on memory:
      //   group 0: mem(0) | mma(0) | mem(1) | mma(1) | ...
      //   group 1:   -    | mem(0) | mma(0) | mem(1) | mma(1) ...
      // Group g reads only rows [g*BM/2, (g+1)*BM/2) of the A tile, kept in
      // its own double buffer, and the whole B tile, kept in a ring of three.
      // In mem(kt) group g loads its A half of tile kt+1 and half of the B
      // rows of tile kt+2; both land before the barrier that ends its mma(kt).
      // A buffers are rewritten two phases after their last reader, B slots
      // three phases after theirs (B(kt+2) replaces B(kt-1)).
      // Naming an accumulation register here makes the compiler select the
      // MFMA form whose accumulator lives in AGPRs: the accumulators then
      // stay out of the VGPR banks that the other wave's LDS reads fill.
      asm volatile("" ::: "a0");
      const int grp = wave >> 2, w4 = wave & 3;
      constexpr int AH = BM / 2;                 // A rows per group
      constexpr int RA2 = AH / 32, RB = NBR / 32, RB2 = RB / 2;
      static_assert(RB % 2 == 0, "B rows split evenly between the groups");
      char* const sAg = smem + grp * 2 * AH * 128;   // this group's A buffers
      char* const sBr = smem + 2 * BM * 128;         // B ring
      const int lrow4 = 8 * w4 + (lane >> 3);
      const int lc4 = swz<8>(lane & 7, lrow4);
      const int mg = m0 + grp * AH;
      const bool fullA = mg + AH <= g.M, fullB = n0 + BN <= g.N;
      const uint32_t vA = (uint32_t)(((int64_t)(mg + lrow4) * g.lda + lc4 * V) * ES);
      const uint32_t vB = (uint32_t)(((int64_t)(n0 + lrow4) * g.ldb + lc4 * V) * ES);
      auto loadA = [&](int kt) {  // this group's A half of tile kt
        const int k0 = kt * BK;
        const bool kok = k0 + lc4 * V < g.K;
        char* d = sAg + (kt & 1) * AH * 128 + w4 * 1024;
#pragma unroll
        for (int i = 0; i < RA2; i++) {
          const bool ok = kok && (fullA || mg + 32 * i + lrow4 < g.M);
          buffer_to_lds16(rA, d + i * 4096, ok ? vA : kOOB, (uint32_t)(32 * i * g.lda * ES + k0 * ES));
        }
      };
      auto loadB = [&](int kt, int half) {  // B rows [half*NBR/2, +NBR/2) of tile kt
        const int k0 = kt * BK;
        const bool kok = k0 + lc4 * V < g.K;
        char* d = sBr + (kt % 3) * NBR * 128 + w4 * 1024;
#pragma unroll
        for (int q = 0; q < RB2; q++) {
          const int i = half * RB2 + q;
          const bool second = DUAL && 32 * i >= BN;
          const int rr = second ? 32 * i - BN : 32 * i;
          const bool ok = kok && (fullB || n0 + rr + lrow4 < g.N);
          buffer_to_lds16(second ? rB3 : rB, d + i * 4096, ok ? vB : kOOB,
                          (uint32_t)(rr * g.ldb * ES + k0 * ES));
        }
      };
      frag afk[KS][MB], bfk[KS][NB], b3k[KS][NB3];
      auto fetch_all = [&](int kt) {
        const char* sA = sAg + (kt & 1) * AH * 128;
        const char* sB = sBr + (kt % 3) * NBR * 128;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const int byte = (ks * M_::KSTEP + lg * M_::E) * ES;
          const int c = byte >> 4, w = byte & 15;
#pragma unroll
          for (int i = 0; i < MB; i++) {
            const int row = wm * WM + i * 32 + lr - grp * AH;  // row within the group's half
            afk[ks][i] = *(const frag*)(sA + row * 128 + (swz<8>(c, row) << 4) + w);
          }
#pragma unroll
          for (int j = 0; j < NB; j++) {
            const int row = wn * WN + j * 32 + lr;
            bfk[ks][j] = *(const frag*)(sB + row * 128 + (swz<8>(c, row) << 4) + w);
            if (DUAL) {
              const int r3 = BN + row;
              b3k[ks][j] = *(const frag*)(sB + r3 * 128 + (swz<8>(c, r3) << 4) + w);
            }
          }
        }
      };
      auto mma_all = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
          for (int i = 0; i < MB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++) {
              acc[i][j] = M_::mma(bfk[ks][j], afk[ks][i], acc[i][j]);
              if (DUAL) acc3[i][j] = M_::mma(b3k[ks][j], afk[ks][i], acc3[i][j]);
            }
      };
      // A workgroup barrier that the compiler neither moves memory
      // operations across nor pairs with waits of its own.
      auto bar = [] {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      if (nk > 0) {
        loadA(0);
        loadB(0, grp);
        if (nk > 1) loadB(1, grp);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        bar();
        if (grp == 1) bar();
        for (int kt = 0; kt < nk; kt++) {
          // (Issuing the fragment reads ahead of the loads measured slower.)
          if (kt + 1 < nk) loadA(kt + 1);
          if (kt + 2 < nk) loadB(kt + 2, grp);
          fetch_all(kt);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          bar();
          __builtin_amdgcn_s_setprio(1);
          mma_all();
          __builtin_amdgcn_s_setprio(0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          // group 1's last phase needs no barrier: no wave waits for it
          if (grp == 0 || kt + 1 < nk) bar();
        }
      }
    } else {
    // Pipeline: tiles kt and kt+1 are resident or in flight while kt computes.
    // The barrier sits before the last k-step's MFMAs: every wave has its
    // fragments of buffer kt in registers (so that buffer may be refilled
    // with tile kt+2) and tile kt+1 has landed (so its first fragments can
    // be read while those MFMAs run).
    if (nk > 0) {
      issue(0, 0);
      if (nk > 1) issue(1, 1);
      if (nk > 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(AC + BC) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      fetch(0, 0, 0);
      for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        compute_head(cur);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // keep the last step's MFMAs below the barrier
        if (kt + 2 < nk) issue(kt + 2, cur);
        if (kt + 1 < nk) fetch(cur ^ 1, 0, LAST ^ 1);
        mfmas(LAST);
        interleave();
        // The next iteration starts from register set 0: move if needed.
        if constexpr (LAST == 0) {
#pragma unroll
          for (int i = 0; i < MB; i++) af[0][i] = af[1][i];
#pragma unroll
          for (int j = 0; j < NB; j++) {
            bfr[0][j] = bfr[1][j];
            if (DUAL) bf3[0][j] = bf3[1][j];
          }
        }
      }
    }
    }
  } else {
    u32x4 ra[AC], rb[BC];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < AC; i++) {
        const int id = tid + NT * i, row = id >> 3, c = id & 7;
        const int gm = m0 + row;
        ra[i] = load_chunk<T, false>(A, gm < g.M, gm, g.lda, k0 + c * V, g.K);
      }
#pragma unroll
      for (int i = 0; i < BC; i++) {
        const int id = tid + NT * i, row = id >> 3, c = id & 7;
        const T* src = B;
        int rr = row;
        if (DUAL && row >= BN) {
          src = B3;
          rr = row - BN;
        }
        const int gn = n0 - nb + rr;
        rb[i] = load_chunk<T, false>(src, gn < nbr, gn, g.ldb, k0 + c * V, g.K);
      }
    };
    auto sstore = [&](int buf) {
      char* sA = smem + buf * STAGE;
      char* sB = sA + BM * 128;
#pragma unroll
      for (int i = 0; i < AC; i++) {
        const int id = tid + NT * i, row = id >> 3, c = id & 7;
        *(u32x4*)(sA + row * 128 + (swz<8>(c, row) << 4)) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < BC; i++) {
        const int id = tid + NT * i, row = id >> 3, c = id & 7;
        *(u32x4*)(sB + row * 128 + (swz<8>(c, row) << 4)) = rb[i];
      }
    };
    if (nk > 0) {
      gload(0);
      sstore(0);
      __syncthreads();
      for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        fetch(cur, 0, 0);
        compute_head(cur);
        mfmas(LAST);
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
      }
    }
  }

  // Epilogue straight from the accumulators: in block (i, j) the lane holds
  // row m = m0 + wm*WM + 32i + lr and, for q = 0..3, the four columns
  // n0 + wn*WN + 32j + 8q + 4lg + {0,1,2,3} in registers 4q..4q+3.
  float* __restrict__ Y = g.Y;
  const T* __restrict__ R = (const T*)g.R;
  T* __restrict__ C = (T*)g.C;
  if constexpr ((EPI == EPI_ACC || EPI == EPI_RESID) && sizeof(T) == 2) {
    // Whole tile inside the matrix, 16-byte aligned rows: the accumulator
    // (and residual) reads of up to four blocks are all issued before the
    // first wait, then their results are stored.  (The memory counter also
    // counts stores, so a block-at-a-time loop pays a full read round trip
    // and a store drain per block.)
    const bool aligned = (g.ldy & 3) == 0 && (EPI != EPI_RESID || ((g.ldr & 3) == 0 && (g.ldc & 3) == 0));
    if (m0 + BM <= g.M && n0 + BN <= g.N && aligned) {
      constexpr int NBLK = MB * NB, HB = NBLK < 4 ? NBLK : 4;
      const bool beta = g.beta != 0;
#pragma unroll
      for (int b0 = 0; b0 < NBLK; b0 += HB) {
        float4 yv[HB][4];
        u32x2 rv[HB][4];
#pragma unroll
        for (int bb = 0; bb < HB; bb++) {
          if (b0 + bb >= NBLK) break;
          const int i = (b0 + bb) / NB, j = (b0 + bb) % NB;
          const int64_t m = m0 + wm * WM + i * 32 + lr;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
            yv[bb][q] = beta ? *(const float4*)(Y + m * g.ldy + n) : make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (EPI == EPI_RESID) rv[bb][q] = *(const u32x2*)(R + m * g.ldr + n);
          }
        }
#pragma unroll
        for (int bb = 0; bb < HB; bb++) {
          if (b0 + bb >= NBLK) break;
          const int i = (b0 + bb) / NB, j = (b0 + bb) % NB;
          const int64_t m = m0 + wm * WM + i * 32 + lr;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
            float s[4] = {yv[bb][q].x + acc[i][j][4 * q], yv[bb][q].y + acc[i][j][4 * q + 1],
                          yv[bb][q].z + acc[i][j][4 * q + 2], yv[bb][q].w + acc[i][j][4 * q + 3]};
            if constexpr (EPI == EPI_RESID) {
              Chunk<T> r;
              r.raw[0] = rv[bb][q][0];
              r.raw[1] = rv[bb][q][1];
#pragma unroll
              for (int e = 0; e < 4; e++) s[e] += to_f(r.e[e]);
              store4<T>(C + m * g.ldc + n, s[0], s[1], s[2], s[3]);
            } else {
              *(float4*)(Y + m * g.ldy + n) = make_float4(s[0], s[1], s[2], s[3]);
            }
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < MB; i++) {
    const int m = m0 + wm * WM + i * 32 + lr;
    if (m >= g.M) continue;
    int64_t pos = m, spos = m;
    int64_t qrows = g.T, krows = g.S;  // Q rows and K/V positions per head
    if constexpr (QKVE) {
      // local row m = b*T + i of sequence b sits at position zigzag(i) of its
      // sequence, key row b*S + zigzag(i)
      const int nbt = g.batch > 0 ? g.batch : 1;
      const int64_t sq = m / g.T;
      spos = zig(m - sq * g.T, g.chunk, g.rank, g.fold);
      pos = sq * g.S + spos;
      qrows = nbt * g.T;
      krows = nbt * g.S;
    }
#pragma unroll
    for (int j = 0; j < NB; j++) {
      float v[16], w[16];
      bool ok[4], full[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
        ok[q] = n < g.N;
        full[q] = n + 3 < g.N;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          v[4 * q + e] = acc[i][j][4 * q + e];
          w[4 * q + e] = 0.f;
        }
      }
      if constexpr (EPI == EPI_ACC || EPI == EPI_RESID) {
        const bool vy = (g.ldy & 3) == 0;
        if (g.beta) {  // gather the accumulator first, then add
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
            const float* py = Y + (int64_t)m * g.ldy + n;
            if (full[q] && vy) {
              const float4 y = *(const float4*)py;
              w[4 * q] = y.x;
              w[4 * q + 1] = y.y;
              w[4 * q + 2] = y.z;
              w[4 * q + 3] = y.w;
            } else if (ok[q]) {
#pragma unroll
              for (int e = 0; e < 4; e++)
                if (n + e < g.N) w[4 * q + e] = py[e];
            }
          }
        }
        if constexpr (EPI == EPI_RESID) {
          const bool vr = (g.ldr & 3) == 0 && (g.ldc & 3) == 0;
          float rr[16];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
            const T* pr = R + (int64_t)m * g.ldr + n;
            if (full[q] && vr) {
              load4<T>(pr, rr + 4 * q);
            } else {
#pragma unroll
              for (int e = 0; e < 4; e++) rr[4 * q + e] = (ok[q] && n + e < g.N) ? to_f(pr[e]) : 0.f;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
            float s[4];
#pragma unroll
            for (int e = 0; e < 4; e++) s[e] = rr[4 * q + e] + w[4 * q + e] + v[4 * q + e];
            T* pc = C + (int64_t)m * g.ldc + n;
            if (full[q] && vr) {
              store4<T>(pc, s[0], s[1], s[2], s[3]);
            } else if (ok[q]) {
#pragma unroll
              for (int e = 0; e < 4; e++)
                if (n + e < g.N) pc[e] = from_f<T>(s[e]);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
            float* py = Y + (int64_t)m * g.ldy + n;
            if (full[q] && vy) {
              *(float4*)py = make_float4(w[4 * q] + v[4 * q], w[4 * q + 1] + v[4 * q + 1],
                                         w[4 * q + 2] + v[4 * q + 2], w[4 * q + 3] + v[4 * q + 3]);
            } else if (ok[q]) {
#pragma unroll
              for (int e = 0; e < 4; e++)
                if (n + e < g.N) py[e] = w[4 * q + e] + v[4 * q + e];
            }
          }
        }
      } else if constexpr (EPI == EPI_STORE) {
        const bool vc = (g.ldc & 3) == 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
          T* pc = C + (int64_t)m * g.ldc + n;
          if (full[q] && vc) {
            store4<T>(pc, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          } else if (ok[q]) {
#pragma unroll
            for (int e = 0; e < 4; e++)
              if (n + e < g.N) pc[e] = from_f<T>(v[4 * q + e]);
          }
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
        const bool vc = (g.ldc & 3) == 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
          float s[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float a = v[4 * q + e];
            const float b = acc3[i][j < NB3 ? j : 0][4 * q + e];
            s[e] = a / (1.0f + fast_exp2(-a * 1.4426950408889634f)) * b;
          }
          T* pc = C + (int64_t)m * g.ldc + n;
          if (full[q] && vc) {
            store4<T>(pc, s[0], s[1], s[2], s[3]);
          } else if (ok[q]) {
#pragma unroll
            for (int e = 0; e < 4; e++)
              if (n + e < g.N) pc[e] = from_f<T>(s[e]);
          }
        }
      } else if constexpr (QKVE) {
        // the 256 x 256 instance is only launched with hd % 32 == 0 and
        // carries the block path alone (the other one costs it registers)
        constexpr bool BLOCK_ONLY = BM == 256 && BN == 256;
        if (BLOCK_ONLY || g.hd % 32 == 0) {
          // The block's 32 columns lie in one head of one part of one shard
          // (hs, ks and the shard width are multiples of hd): split the
          // block's first column once, from a wave-uniform value, and step
          // through the block by offsets.
          int c = __builtin_amdgcn_readfirstlane(n0 + wn * WN + j * 32 + g.col0);
          T* qb = (T*)g.Q;
          T* kb = (T*)g.Kd;
          T* vb = (T*)g.Vt;
          if (g.shard_cols > 0) {
            const int u = c / g.shard_cols;
            c -= u * g.shard_cols;
            qb += u * g.q_stride;
            kb += u * g.kv_stride;
            vb += u * g.kv_stride;
          }
          const int part = c < g.hs ? 0 : (c < g.hs + g.ks ? 1 : 2);
          const int rem = part == 0 ? c : c - g.hs - (part - 1) * g.ks;
          const int head = rem / g.hd;
          const int e0 = rem - head * g.hd;
          T* const qrow = qb + ((int64_t)head * qrows + m) * g.hd + e0;
          T* const krow = kb + ((int64_t)head * krows + pos) * g.hd + e0;
          T* const vcol = vb + ((int64_t)head * g.hd + e0) * krows + pos;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            if (!ok[q]) continue;
            const int eo = 8 * q + 4 * lg;  // the chunk's first column within the block
            float o4[4] = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            if constexpr (ROPE)
              if (part < 2) rope_pairs(o4, e0 + eo, spos, g.rope_l2 / g.hd);
            if (part == 0) {
              store4<T>(qrow + eo, o4[0], o4[1], o4[2], o4[3]);
            } else if (part == 1) {
              store4<T>(krow + eo, o4[0], o4[1], o4[2], o4[3]);
            } else {
              T* pv = vcol + (int64_t)eo * krows;
#pragma unroll
              for (int t = 0; t < 4; t++) pv[(int64_t)t * krows] = from_f<T>(o4[t]);
            }
          }
          continue;
        }
        if constexpr (!BLOCK_ONLY) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          if (!ok[q]) continue;
          const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
          // hs, ks and hd are multiples of 4, so the four columns share shard, part and head.
          int c = n + g.col0;
          T* qb = (T*)g.Q;
          T* kb = (T*)g.Kd;
          T* vb = (T*)g.Vt;
          if (g.shard_cols > 0) {
            const int u = c / g.shard_cols;
            c -= u * g.shard_cols;
            qb += u * g.q_stride;
            kb += u * g.kv_stride;
            vb += u * g.kv_stride;
          }
          const int part = c < g.hs ? 0 : (c < g.hs + g.ks ? 1 : 2);
          const int rem = part == 0 ? c : c - g.hs - (part - 1) * g.ks;
          const int head = rem / g.hd;
          const int e = rem - head * g.hd;
          float o4[4] = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
          if constexpr (ROPE)
            if (part < 2) rope_pairs(o4, e, spos, g.rope_l2 / g.hd);
          if (part == 0) {
            store4<T>(qb + ((int64_t)head * qrows + m) * g.hd + e, o4[0], o4[1], o4[2], o4[3]);
          } else if (part == 1) {
            store4<T>(kb + ((int64_t)head * krows + pos) * g.hd + e, o4[0], o4[1], o4[2], o4[3]);
          } else {
            T* pv = vb + ((int64_t)head * g.hd + e) * krows + pos;
#pragma unroll
            for (int t = 0; t < 4; t++) pv[(int64_t)t * krows] = from_f<T>(o4[t]);
          }
        }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Zigzag-aware causal flash attention of the local queries of one head group
// against the gathered K/V.
//
// A work item is (head, query tile of kBQ local rows, key segment).  Each of
// the 4 waves owns kQB blocks of 32 queries (every K or V^T fragment read
// from LDS feeds kQB MFMAs); with kQB = 1 two workgroups share a CU, so one
// wave's softmax overlaps the other's MFMAs.  K/V tiles of 64 keys go
// straight from global memory into LDS (double-buffered, one barrier per
// tile); keys at or past the item's last query position + 1 read as zero,
// so rows the rank never receives are never used.  Per tile a wave computes
// S^T = K . Q^T (lane <-> query, registers <-> keys), masks only tiles that
// reach past its smallest query position, and accumulates O^T += V^T . P^T
// with P kept in registers.  Softmax runs in log2 units with the scale
// folded into one FMA; the running max used for the exponentials is only
// raised (rescaling O and the running sum) when a new score exceeds it by
// more than 2^8, which keeps every exponential <= 2^8 while skipping almost
// all rescales.  K rows are fed to the first product in an order that swaps
// bits 2 and 3 of the row index, which makes each lane hold 8 consecutive
// keys per 16-key step of P, so the matching V^T operand is one 16-byte LDS
// read.
//
// Query tiles whose key range exceeds the segment length are split into
// several items; their partial (max, sum, unnormalised O) are merged by
// attn_combine_kernel.  Items are ordered heaviest first, and
// head = item % Hd keeps one head on each XCD when Hd divides 8.
//
// attn_kernel serves fp32 and the head dims other than 128; bf16 with
// 128-dim heads runs the software-pipelined attn_pipe_kernel further down
// (same items, tiles and layouts).
// ---------------------------------------------------------------------------
constexpr int kQB = 1;     // 32-query blocks per wave (two waves share a SIMD)
constexpr int kBQ = 128 * kQB;  // local query rows per work item (4 waves)
constexpr int kBQW = 256;       // the same for attn_pipe_kernel<8> (8 waves)
#ifndef TSP_ATTN_WIDE
#define TSP_ATTN_WIDE 1         // bf16 128-dim attention on 256-row tiles (0: 128-row tiles, 4 waves)
#endif
constexpr int kBKV = 64;   // keys per tile

// Keys per K/V tile and LDS stages of attn_kernel: 64-key tiles, double
// buffered (the 128-dim bf16 instance is only used when the pipelined kernel
// is switched off).
#ifndef TSP_ATTN128_BKV
#define TSP_ATTN128_BKV 64   // keys per tile of the 128-dim bf16 kernel
#endif
#ifndef TSP_ATTN_VPRE
#define TSP_ATTN_VPRE 2      // 16-key steps of V^T fragments read before the softmax
#endif
#ifndef TSP_ATTN128_WAVES
#define TSP_ATTN128_WAVES 2  // waves per SIMD the 128-dim bf16 kernel is sized for
#endif
template <typename T, int HD>
struct AttnTile {
  static constexpr bool deep = sizeof(T) == 2 && HD == 128;
  static constexpr int BKV = deep ? TSP_ATTN128_BKV : 64;
  static constexpr int NSTAGE = 2;
  static constexpr int WAVES = deep ? TSP_ATTN128_WAVES : 2;  // waves per SIMD
};

// Does the key tile starting at k0 lie in one of the rank's own chunks
// (r and 2D-1-r), whose K/V rows come from the rank's own buffer when the
// other ranks' rows are read in place?
struct OwnChunks {
  int lo1, hi1, lo2, hi2;
  __device__ __attribute__((always_inline)) OwnChunks(const AttnArgs& a) {
    const int c = (int)a.chunk;
    lo1 = a.rank * c;
    hi1 = lo1 + c;
    lo2 = (2 * a.fold - 1 - a.rank) * c;
    hi2 = lo2 + c;
  }
  __device__ bool operator()(int k0) const {
    return (k0 >= lo1 && k0 < hi1) || (k0 >= lo2 && k0 < hi2);
  }
};

__device__ inline int kappa(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }



// One past the causal end of query tile qt (bq local rows per tile).
__device__ __host__ inline int64_t qtile_kend(int64_t T, int qt, int64_t C, int rank, int fold, int bq) {
  const int64_t last = (T < (int64_t)qt * bq + bq ? T : (int64_t)qt * bq + bq) - 1;
  return zig(last, C, rank, fold) + 1;
}

// Work items are dispatched segment-major: every query tile's first key
// segment, then every tile's second, ... (heaviest tiles first within a
// segment), so the workgroups in flight read the same key range and share it
// in L2.  Query tile qt has a segment s iff its causal end kend(qt) > s*lseg;
// kend grows with qt, so those tiles form a suffix [q0(s), nqt).
__device__ __attribute__((always_inline)) inline int first_tile_past(const AttnArgs& a, int64_t lo) {
  int l = 0, h = a.nqt;  // smallest qt with kend(qt) > lo
  while (l < h) {
    const int mid = (l + h) >> 1;
    if (qtile_kend(a.T, mid, a.chunk, a.rank, a.fold, a.bq) > lo)
      h = mid;
    else
      l = mid + 1;
  }
  return l;
}

// Micro-batch: sequences of one call (0 means 1).
__device__ __host__ inline int batch_of(const AttnArgs& a) { return a.batch > 0 ? a.batch : 1; }

// K/V head read by query head `head` (grouped-query attention).
__device__ __attribute__((always_inline)) inline int kv_head(const AttnArgs& a, int head) {
  return a.grp > 1 ? head / a.grp : head;
}

// Offset (elements) of K/V head kvh's shard in K, Vt, Kg and Vtg; kvh becomes
// the head's index within its shard.
__device__ __attribute__((always_inline)) inline int64_t kv_shard_base(const AttnArgs& a, int& kvh) {
  if (a.kvh_per_shard <= 0) return 0;
  const int u = kvh / a.kvh_per_shard;
  kvh -= u * a.kvh_per_shard;
  return (int64_t)u * a.shard_stride;
}

// Workgroup -> (head, sequence sb, work item): heads innermost, then the
// sequences of the micro-batch, then the items.
__device__ __attribute__((always_inline)) inline void block_item(const AttnArgs& a, int& head, int& sb,
                                                                 int& item) {
  const int nb = batch_of(a);
  head = blockIdx.x % a.Hd;
  const int r = blockIdx.x / a.Hd;
  sb = r % nb;
  item = r / nb;
}

__device__ __attribute__((always_inline)) inline bool decode_item(const AttnArgs& a, int item, int& qt, int& seg, int& nseg,
                                   int64_t& kend) {
  for (seg = 0; seg < a.maxseg; seg++) {
    const int cnt = a.nqt - first_tile_past(a, (int64_t)seg * a.lseg);
    if (item < cnt) {
      qt = a.nqt - 1 - item;
      kend = qtile_kend(a.T, qt, a.chunk, a.rank, a.fold, a.bq);
      nseg = (int)((kend + a.lseg - 1) / a.lseg);
      return true;
    }
    item -= cnt;
  }
  return false;
}

template <typename T, int HD>
__global__ void __launch_bounds__(256, (kQB == 1 ? AttnTile<T, HD>::WAVES : 1)) attn_kernel(AttnArgs a) {
  typedef MF<T> M_;
  typedef typename M_::frag frag;
  constexpr int ES = sizeof(T);
  constexpr int V = 16 / ES;
  constexpr int QB = kQB;
  constexpr int BKV = AttnTile<T, HD>::BKV;
  constexpr int NSTAGE = AttnTile<T, HD>::NSTAGE;
  constexpr int NKB = BKV / 32;         // 32-key blocks per tile
  constexpr int KROWB = HD * ES, KCH = KROWB / 16;
  constexpr int VROWB = BKV * ES, VCH = VROWB / 16;
  constexpr int KT_BYTES = BKV * KROWB;
  constexpr int VT_BYTES = HD * VROWB;
  constexpr int STAGE = KT_BYTES + VT_BYTES;
  constexpr int KI = KT_BYTES / 1024, VI = VT_BYTES / 1024;  // 1 KB wave loads per tile
  constexpr int QK = HD / M_::KSTEP;    // k-steps over the head dim
  constexpr int DB = (HD + 31) / 32;    // 32-row blocks of O^T
  constexpr int PK = BKV / M_::KSTEP;   // k-steps over the keys of a tile
  static_assert(KT_BYTES % 1024 == 0 && VT_BYTES % 1024 == 0, "tile bytes");
  static_assert(NSTAGE == 2 || (KI % 4 == 0 && VI % 4 == 0), "deep rings need equal loads per wave");
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  int head, sb, item;
  block_item(a, head, sb, item);
  int qt, seg, nseg;
  int64_t kend;
  if (!decode_item(a, item, qt, seg, nseg, kend)) return;
  // sequence sb: its local rows, its key rows and the V^T row stride
  const int nb = batch_of(a);
  const int64_t BS = (int64_t)nb * a.S, BT = (int64_t)nb * a.T;

  // Positions fit in 32 bits (S < 2^31).
  const int kend32 = (int)kend;
  const int kbeg = seg * a.lseg;
  const int kfin = min(kend32, kbeg + a.lseg);
  const int T32 = (int)a.T;
  const int row0 = qt * kBQ + wave * 32 * QB;  // this wave's first local row
  const int C32 = (int)a.chunk;
  int qpos[QB];
  bool qok[QB];
#pragma unroll
  for (int b = 0; b < QB; b++) {
    const int row = row0 + 32 * b + lr;
    qok[b] = row < T32;
    qpos[b] = qok[b] ? (int)zig(row, C32, a.rank, a.fold) : -1;
  }
  const bool wok = row0 < T32;
  const bool wfull = row0 + 32 * QB - 1 < T32;
  const int kend_w = wok ? (int)zig(min(T32, row0 + 32 * QB) - 1, C32, a.rank, a.fold) + 1 : 0;
  const int qmin_w = wok ? (int)zig(row0, C32, a.rank, a.fold) : 0;

  int kvh = kv_head(a, head);
  const int64_t kvb = kv_shard_base(a, kvh);
  const T* Qh = (const T*)a.Q + ((int64_t)head * BT + (int64_t)sb * a.T) * HD;
  const T* Kh = (const T*)a.K + kvb + ((int64_t)kvh * BS + (int64_t)sb * a.S) * HD;
  const T* Vh = (const T*)a.Vt + kvb + (int64_t)kvh * HD * BS + (int64_t)sb * a.S;

  frag qf[QB][QK];
#pragma unroll
  for (int b = 0; b < QB; b++)
#pragma unroll
    for (int ks = 0; ks < QK; ks++) {
      const int e0 = ks * M_::KSTEP + lg * M_::E;
      if (qok[b])
        qf[b][ks] = *(const frag*)(Qh + (row0 + 32 * b + lr) * HD + e0);
      else
        qf[b][ks] = frag{0};
    }

  f32x16 o[QB][DB];
#pragma unroll
  for (int b = 0; b < QB; b++)
#pragma unroll
    for (int d = 0; d < DB; d++) o[b][d] = f32x16{0};
  float m[QB], l[QB];
#pragma unroll
  for (int b = 0; b < QB; b++) {
    m[b] = -INFINITY;
    l[b] = 0.f;
  }

  // Direct loads.  Wave-load ii of the K tile fills LDS bytes
  // [ii*1024, ii*1024+1024): lane l writes 16 bytes at physical chunk p of
  // row r, holding logical chunk p ^ (r % KCH) of key k0 + r.  Likewise for
  // V^T rows d (64 keys each).
  const bool split_src = a.Kg != nullptr;
  const OwnChunks own_tile(a);
  const T* Kgh = split_src ? (const T*)a.Kg + kvb + ((int64_t)kvh * BS + (int64_t)sb * a.S) * HD : Kh;
  const T* Vgh = split_src ? (const T*)a.Vtg + kvb + (int64_t)kvh * HD * BS + (int64_t)sb * a.S : Vh;
  constexpr int KJ = (KI + 3) / 4, VJ = (VI + 3) / 4;  // wave loads per tile per wave
  int krow[KJ], voff[VJ], vkey[VJ];
  uint32_t koff[KJ];
#pragma unroll
  for (int j = 0; j < KJ; j++) {
    const int b = (wave + 4 * j) * 1024 + 16 * lane;
    const int r = b / KROWB, p = (b % KROWB) >> 4;
    krow[j] = r;
    koff[j] = (uint32_t)((r * HD + swz<KCH>(p, r) * V) * ES);
  }
#pragma unroll
  for (int j = 0; j < VJ; j++) {
    const int b = (wave + 4 * j) * 1024 + 16 * lane;
    const int d = b / VROWB, p = (b % VROWB) >> 4;
    const int c = swz<VCH>(p, d);
    vkey[j] = c * V;
    voff[j] = (int)(((int64_t)d * BS + c * V) * ES);
  }
  // This wave's KJ + VJ loads of a tile (K first).
  auto issue = [&](int k0, int buf) {
    char* sK = smem + buf * STAGE;
    char* sV = sK + KT_BYTES;
    const bool mine = !split_src || own_tile(k0);
    const brsrc rK = make_rsrc(mine ? Kh : Kgh, (uint64_t)a.S * HD * ES);
    const brsrc rV = make_rsrc(mine ? Vh : Vgh, (uint64_t)((HD - 1) * BS + a.S) * ES);
#pragma unroll
    for (int j = 0; j < KJ; j++) {
      if (KI % 4 == 0 || wave + 4 * j < KI)
        buffer_to_lds16(rK, sK + (wave + 4 * j) * 1024, k0 + krow[j] < kend32 ? koff[j] : kOOB,
                        (uint32_t)(k0 * HD * ES));
    }
#pragma unroll
    for (int j = 0; j < VJ; j++) {
      if (VI % 4 == 0 || wave + 4 * j < VI)
        buffer_to_lds16(rV, sV + (wave + 4 * j) * 1024,
                        k0 + vkey[j] < kend32 ? (uint32_t)voff[j] : kOOB, (uint32_t)(k0 * ES));
    }
  };
  // A V^T chunk that straddles kend was loaded whole: zero its keys >= kend.
  auto fixup = [&](int k0, int buf) {
    char* sV = smem + buf * STAGE + KT_BYTES;
    const int first = kend32 - k0;  // first key to clear, within the tile
    const int upto = min(BKV, (first + V - 1) / V * V);
    for (int i = tid; i < HD * (upto - first); i += 256) {
      const int d = i / (upto - first), key = first + i % (upto - first);
      const int byte = key * ES;
      const int c = byte >> 4, w = byte & 15;
      *(T*)(sV + d * VROWB + (swz<VCH>(c, d) << 4) + w) = from_f<T>(0.f);
    }
  };

  const float cs = a.scale_log2;
  auto compute = [&](int buf, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* sK = smem + buf * STAGE;
    const char* sV = sK + KT_BYTES;
    f32x16 s[QB][NKB];
    __builtin_amdgcn_s_setprio(1);  // raise wave priority around MFMA blocks
#pragma unroll
    for (int kb = 0; kb < NKB; kb++) {
#pragma unroll
      for (int b = 0; b < QB; b++) s[b][kb] = f32x16{0};
      const int krow = 32 * kb + kappa(lr);
#pragma unroll
      for (int ks = 0; ks < QK; ks++) {
        const int byte = (ks * M_::KSTEP + lg * M_::E) * ES;
        const int c = byte >> 4, w = byte & 15;
        const frag kf = *(const frag*)(sK + krow * KROWB + (swz<KCH>(c, krow) << 4) + w);
#pragma unroll
        for (int b = 0; b < QB; b++) s[b][kb] = M_::mma(kf, qf[b][ks], s[b][kb]);
      }
    }
    // Keep each fragment read one step ahead of the MFMAs that use it.
#pragma unroll
    for (int q = 0; q < NKB * QK; q++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // V^T fragments of the whole tile, read while the products above run
    // and the softmax below computes (the K fragments' registers are free).
    auto vfrag = [&](int st, int d) {
      int kk;  // first key (within the tile) this lane supplies at step st
      if constexpr (M_::E == 8) {
        kk = 16 * st + 8 * lg;
      } else {
        const int i = st & 15;
        kk = 32 * (st >> 4) + 16 * (i >> 3) + 8 * lg + (i & 7);
      }
      const int byte = kk * ES;
      const int c = byte >> 4, w = byte & 15;
      const int drow = 32 * d + lr;
      if (HD % 32 == 0 || drow < HD)
        return *(const frag*)(sV + drow * VROWB + (swz<VCH>(c, drow) << 4) + w);
      return frag{0};
    };
    constexpr int NVP = TSP_ATTN_VPRE < PK ? TSP_ATTN_VPRE : PK;  // steps read early
    frag vpre[NVP > 0 ? NVP : 1][DB];
#pragma unroll
    for (int st = 0; st < NVP; st++)
#pragma unroll
      for (int d = 0; d < DB; d++) vpre[st][d] = vfrag(st, d);
    if constexpr (NVP > 0) __builtin_amdgcn_sched_barrier(0);
    // Register i of block kb holds key k0 + 32kb + 16(i/8) + 8lg + i%8.
    float mt[QB];
#pragma unroll
    for (int b = 0; b < QB; b++) {
      // four independent max chains (short dependency paths)
      float xs[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      // key - k0 - 8lg = 32kb + 16(i/8) + i%8 must not exceed qpos - k0 - 8lg
      const int lim = max(-1, min(BKV, qpos[b] - k0)) - 8 * lg;
#pragma unroll
      for (int kb = 0; kb < NKB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          if (MASK) {
            if (32 * kb + 16 * (i >> 3) + (i & 7) > lim) s[b][kb][i] = -INFINITY;
          }
          xs[i & 3] = fmaxf(xs[i & 3], s[b][kb][i]);
        }
      float x = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3]));
      x = halves_max(x);
      mt[b] = x * cs;  // log2 units (scale > 0, so -inf stays -inf)
    }
    bool grow = false;
#pragma unroll
    for (int b = 0; b < QB; b++) grow |= mt[b] > m[b] + 8.0f;
    if (__any(grow)) {
#pragma unroll
      for (int b = 0; b < QB; b++) {
        const float mn = fmaxf(m[b], mt[b]);
        const float alpha = m[b] == -INFINITY ? 0.f : fast_exp2(m[b] - mn);
        m[b] = mn;
        l[b] *= alpha;
#pragma unroll
        for (int d = 0; d < DB; d++) o[b][d] *= alpha;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    frag pf[QB][PK];
#pragma unroll
    for (int b = 0; b < QB; b++) {
      const float nm = m[b] == -INFINITY ? 0.f : -m[b];
      float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four independent sum chains
#pragma unroll
      for (int st = 0; st < PK; st++) {
        if constexpr (M_::E == 8) {
          const int kb = st >> 1, i0 = (st & 1) * 8;
#pragma unroll
          for (int t = 0; t < 8; t++) {
            const float p = fast_exp2(fmaf(s[b][kb][i0 + t], cs, nm));
            ls[t & 3] += p;
            pf[b][st][t] = (bf16)p;
          }
        } else {
          const float p = fast_exp2(fmaf(s[b][st >> 4][st & 15], cs, nm));
          ls[st & 3] += p;
          pf[b][st] = p;
        }
      }
      l[b] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T . P^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < PK; st++) {
#pragma unroll
      for (int d = 0; d < DB; d++) {
        const frag vf = st < NVP ? vpre[st < NVP ? st : 0][d] : vfrag(st, d);
#pragma unroll
        for (int b = 0; b < QB; b++) o[b][d] = M_::mma(vf, pf[b][st], o[b][d]);
      }
    }
    if constexpr (NVP == 0) {
#pragma unroll
      for (int q = 0; q < PK * DB; q++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 2);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  const int ntiles = (kfin - kbeg + BKV - 1) / BKV;
  // Prologue: tiles 0 .. NSTAGE-2 in flight.
#pragma unroll
  for (int t = 0; t < NSTAGE - 1; t++)
    if (t < ntiles) issue(kbeg + t * BKV, t);
  for (int t = 0; t < ntiles; t++) {
    const int k0 = kbeg + t * BKV;
    // Wait for this tile's loads: loads retire in order, and each wave has
    // issued LPT loads for each of the (at most NSTAGE-2) later tiles.
    if constexpr (NSTAGE == 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      constexpr int LPT = (KI + VI) / 4;
      const int later = min(NSTAGE - 2, ntiles - 1 - t);
      static_assert(NSTAGE == 4 && LPT == 4, "wait counts below assume 4 loads per tile");
      if (later >= 2)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (later == 1)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (k0 + BKV > kend32 && (kend32 % V) != 0) {  // last tile, V^T chunk straddles kend
      fixup(k0, t % NSTAGE);
      __syncthreads();
    }
    const bool more = t + NSTAGE - 1 < ntiles;
    const int nk0 = more ? k0 + (NSTAGE - 1) * BKV : -1, nbuf = (t + NSTAGE - 1) % NSTAGE;
    if (more) issue(nk0, nbuf);
    if (k0 < kend_w) {
      if (!wfull || k0 + BKV - 1 > qmin_w)
        compute(t % NSTAGE, k0, std::true_type{});
      else
        compute(t % NSTAGE, k0, std::false_type{});
    }
  }

#pragma unroll
  for (int b = 0; b < QB; b++) {
    const float lt = halves_sum(l[b]);
    const int64_t row = row0 + 32 * b + lr;
    (void)kend_w;
    if (nseg == 1) {
      if (qok[b]) {
        const float inv = 1.0f / lt;
        if (a.LSE && lg == 0) a.LSE[((int64_t)head * nb + sb) * a.T + row] = m[b] + log2f(lt);
        T* orow = (T*)a.O + ((int64_t)sb * a.T + row) * a.ldo + head * HD;
#pragma unroll
        for (int d = 0; d < DB; d++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int d0 = 32 * d + 8 * q + 4 * lg;
            if (HD % 32 == 0 || d0 < HD)
              store4<T>(orow + d0, o[b][d][4 * q] * inv, o[b][d][4 * q + 1] * inv,
                        o[b][d][4 * q + 2] * inv, o[b][d][4 * q + 3] * inv);
          }
      }
    } else {
      const int64_t slot =
          ((((int64_t)head * nb + sb) * a.nqt + qt) * a.maxseg + seg) * kBQ + wave * 32 * QB + 32 * b + lr;
      float* op = a.Op + slot * HD;
#pragma unroll
      for (int d = 0; d < DB; d++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int d0 = 32 * d + 8 * q + 4 * lg;
          if (HD % 32 == 0 || d0 < HD)
            *(float4*)(op + d0) =
                make_float4(o[b][d][4 * q], o[b][d][4 * q + 1], o[b][d][4 * q + 2], o[b][d][4 * q + 3]);
        }
      if (lg == 0) {
        a.ML[2 * slot] = m[b];
        a.ML[2 * slot + 1] = lt;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined attention for bf16 with 128-dim heads.  Same tiles,
// LDS layouts, masking and softmax as attn_kernel (one wave per 32 queries,
// 64-key tiles), on NW waves per workgroup: NW = 8 (the default) takes
// 256-row query tiles, one workgroup per CU, so each K/V tile brought into
// LDS serves twice the rows of NW = 4 (128-row tiles, two workgroups per
// CU) and the global-to-LDS loads per flop halve; both run two waves per
// SIMD.  Each wave overlaps its own MFMAs with its softmax instead of
// alternating between them:
//   phase A of tile t:  S(t+1) = K(t+1) . Q^T      with the exponentials of
//                                                  tile t's second 32 keys
//   phase B of tile t:  O^T += V^T(t) . P^T(t)     with the exponentials of
//                                                  tile t+1's first 32 keys
// The row max of S(t+1) is taken between the phases; the lazy rescale of O
// (same 2^8 rule) is applied after phase B, once tile t's products are in.
// K runs one tile ahead of V^T, so each has its own pair of LDS buffers:
// iteration t reads K(t+1) and V^T(t) and loads K(t+2) and V^T(t+1), one
// barrier per tile as before.
// ---------------------------------------------------------------------------
#ifndef TSP_PIPE_DIST
#define TSP_PIPE_DIST 3    // LDS fragment reads kept in flight ahead of the MFMAs
#endif
#ifndef TSP_ATTN_SPREAD
#define TSP_ATTN_SPREAD 0  // the next tiles' loads spread over phase A (below)
#endif
#ifndef TSP_ATTN_FOLD
#define TSP_ATTN_FOLD 1    // softmax scale and offset folded into the S products (below)
#endif

template <int NW>
__global__ void __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) attn_pipe_kernel(AttnArgs a) {
  typedef bf16 T;
  typedef MF<bf16> M_;
  typedef bf16x8 frag;
  static_assert(kQB == 1 && (NW == 4 || NW == 8), "one 32-query block per wave");
  constexpr int BQ = 32 * NW;  // local query rows per work item
  constexpr int HD = 128, ES = 2, V = 8, BKV = 64;
  constexpr int KROWB = HD * ES, KCH = KROWB / 16;   // K rows: 256 B
  constexpr int VROWB = BKV * ES, VCH = VROWB / 16;  // V^T rows: 128 B
  constexpr int KT = BKV * KROWB, VT = HD * VROWB;   // 16 KB per tile each
  constexpr int QK = HD / 16, DB = HD / 32, PK = BKV / 16;
  constexpr int KJ = KT / (NW * 1024), VJ = VT / (NW * 1024);  // 1 KB loads per wave per tile
  static_assert(KJ + VJ <= 8, "spread loads: one per second MFMA of phase A");
  __shared__ __attribute__((aligned(16))) char smem[2 * KT + 2 * VT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  int head, sb, item;
  block_item(a, head, sb, item);
  int qt, seg, nseg;
  int64_t kend;
  if (!decode_item(a, item, qt, seg, nseg, kend)) return;
  // sequence sb: its local rows, its key rows and the V^T row stride
  const int nb = batch_of(a);
  const int64_t BS = (int64_t)nb * a.S, BT = (int64_t)nb * a.T;
  const int kend32 = (int)kend;
  const int kbeg = seg * a.lseg;
  const int kfin = min(kend32, kbeg + a.lseg);
  const int T32 = (int)a.T, C32 = (int)a.chunk;
  const int row0 = qt * BQ + wave * 32;
  const bool qok = row0 + lr < T32;
  const int qpos = qok ? (int)zig(row0 + lr, C32, a.rank, a.fold) : -1;
  const bool wok = row0 < T32;
  const bool wfull = row0 + 31 < T32;
  const int kend_w = wok ? (int)zig(min(T32, row0 + 32) - 1, C32, a.rank, a.fold) + 1 : 0;
  const int qmin_w = wok ? (int)zig(row0, C32, a.rank, a.fold) : 0;

  int kvh = kv_head(a, head);
  const int64_t kvb = kv_shard_base(a, kvh);
  const T* Qh = (const T*)a.Q + ((int64_t)head * BT + (int64_t)sb * a.T) * HD;
  const T* Kh = (const T*)a.K + kvb + ((int64_t)kvh * BS + (int64_t)sb * a.S) * HD;
  const T* Vh = (const T*)a.Vt + kvb + (int64_t)kvh * HD * BS + (int64_t)sb * a.S;
  frag qf[QK];
#pragma unroll
  for (int ks = 0; ks < QK; ks++)
    qf[ks] = qok ? *(const frag*)(Qh + (int64_t)(row0 + lr) * HD + ks * 16 + lg * 8) : frag{0};

  // Direct loads, as in attn_kernel.
  const bool split_src = a.Kg != nullptr;
  const OwnChunks own_tile(a);
  const T* Kgh = split_src ? (const T*)a.Kg + kvb + ((int64_t)kvh * BS + (int64_t)sb * a.S) * HD : Kh;
  const T* Vgh = split_src ? (const T*)a.Vtg + kvb + (int64_t)kvh * HD * BS + (int64_t)sb * a.S : Vh;
  int krow[KJ], vkey[VJ];
  uint32_t koff[KJ], voff[VJ];
#pragma unroll
  for (int j = 0; j < KJ; j++) {
    const int b = (wave + NW * j) * 1024 + 16 * lane;
    const int r = b / KROWB, p = (b % KROWB) >> 4;
    krow[j] = r;
    koff[j] = (uint32_t)((r * HD + swz<KCH>(p, r) * V) * ES);
  }
#pragma unroll
  for (int j = 0; j < VJ; j++) {
    const int b = (wave + NW * j) * 1024 + 16 * lane;
    const int d = b / VROWB, p = (b % VROWB) >> 4;
    const int c = swz<VCH>(p, d);
    vkey[j] = c * V;
    voff[j] = (uint32_t)(((int64_t)d * BS + c * V) * ES);
  }
  char* const sK0 = smem;
  char* const sV0 = smem + 2 * KT;
  // The wave's 1 KB slice of each tile, as a wave-uniform (scalar) offset so
  // that the LDS destinations are formed without per-load VALU work.
  const int wofs = __builtin_amdgcn_readfirstlane(wave * 1024);
  // Tiles wholly below kend need no per-lane range selects.
  auto issueK = [&](int k0, int buf) {
    const brsrc rK = make_rsrc(!split_src || own_tile(k0) ? Kh : Kgh, (uint64_t)a.S * HD * ES);
    if (k0 + BKV <= kend32) {
#pragma unroll
      for (int j = 0; j < KJ; j++)
        buffer_to_lds16(rK, sK0 + buf * KT + wofs + NW * 1024 * j, koff[j], (uint32_t)(k0 * HD * ES));
    } else {
#pragma unroll
      for (int j = 0; j < KJ; j++)
        buffer_to_lds16(rK, sK0 + buf * KT + wofs + NW * 1024 * j,
                        k0 + krow[j] < kend32 ? koff[j] : kOOB, (uint32_t)(k0 * HD * ES));
    }
  };
  auto issueV = [&](int k0, int buf) {
    const brsrc rV = make_rsrc(!split_src || own_tile(k0) ? Vh : Vgh, (uint64_t)((HD - 1) * BS + a.S) * ES);
    if (k0 + BKV <= kend32) {
#pragma unroll
      for (int j = 0; j < VJ; j++)
        buffer_to_lds16(rV, sV0 + buf * VT + wofs + NW * 1024 * j, voff[j], (uint32_t)(k0 * ES));
    } else {
#pragma unroll
      for (int j = 0; j < VJ; j++)
        buffer_to_lds16(rV, sV0 + buf * VT + wofs + NW * 1024 * j,
                        k0 + vkey[j] < kend32 ? voff[j] : kOOB, (uint32_t)(k0 * ES));
    }
  };
  // One of the wave's KJ (VJ) loads of a K (V^T) tile.
  auto issueK1 = [&](int k0, int buf, int j) {
    const brsrc rK = make_rsrc(!split_src || own_tile(k0) ? Kh : Kgh, (uint64_t)a.S * HD * ES);
    buffer_to_lds16(rK, sK0 + buf * KT + wofs + NW * 1024 * j,
                    k0 + BKV <= kend32 || k0 + krow[j] < kend32 ? koff[j] : kOOB, (uint32_t)(k0 * HD * ES));
  };
  auto issueV1 = [&](int k0, int buf, int j) {
    const brsrc rV = make_rsrc(!split_src || own_tile(k0) ? Vh : Vgh, (uint64_t)((HD - 1) * BS + a.S) * ES);
    buffer_to_lds16(rV, sV0 + buf * VT + wofs + NW * 1024 * j,
                    k0 + BKV <= kend32 || k0 + vkey[j] < kend32 ? voff[j] : kOOB, (uint32_t)(k0 * ES));
  };
  auto fixupV = [&](int k0, int buf) {
    char* sV = sV0 + buf * VT;
    const int first = kend32 - k0;
    const int upto = min(BKV, (first + V - 1) / V * V);
    for (int i = tid; i < HD * (upto - first); i += 64 * NW) {
      const int d = i / (upto - first), key = first + i % (upto - first);
      const int byte = key * ES;
      *(T*)(sV + d * VROWB + (swz<VCH>(byte >> 4, d) << 4) + (byte & 15)) = from_f<T>(0.f);
    }
  };
  // K fragment of 32-key block kb, k-step ks (rows fed in kappa order) and
  // V^T fragment of d-block d, 16-key step st.
  // The lane-dependent part of each fragment address is computed once; the
  // buffer, block and d offsets are compile-time and become the reads'
  // immediate offsets (the swizzle terms do not depend on them: 32-row blocks
  // leave r % 16 and (r / 2) % 8 unchanged).
  int koffl[QK], voffl[PK];
#pragma unroll
  for (int ks = 0; ks < QK; ks++)
    koffl[ks] = kappa(lr) * KROWB + (swz<KCH>(2 * ks + lg, kappa(lr)) << 4);
#pragma unroll
  for (int st = 0; st < PK; st++) voffl[st] = lr * VROWB + (swz<VCH>(2 * st + lg, lr) << 4);
  auto kfrag = [&](int buf, int kb, int ks) {
    return *(const frag*)(sK0 + buf * KT + kb * 32 * KROWB + koffl[ks]);
  };
  auto vfrag = [&](int buf, int st, int d) {
    return *(const frag*)(sV0 + buf * VT + d * 32 * VROWB + voffl[st]);
  };

  const float cs = a.scale_log2;
  const float kSumCap = a.sum_cap;
  // Folded softmax offset.  The wave's queries are prescaled by cs, so scores
  // arrive in log2 units, and every 32-key S block starts with one extra MFMA
  // of a constant K fragment (a one at k = 0 in every key row) and a query
  // fragment holding -m at k = 0 (m: the row's reference max, kept
  // representable in bf16).  The block then holds s*cs - m and feeds the
  // exponentials as it is: the per-score FMA moves onto the matrix unit, two
  // MFMAs per 64-key tile.  S blocks already formed when m is raised are
  // shifted by the change.
  constexpr bool FOLD = TSP_ATTN_FOLD != 0;
  frag kext = frag{0}, qext = frag{0};
  if constexpr (FOLD) {
    if (lg == 0) kext[0] = (bf16)1.0f;
#pragma unroll
    for (int ks = 0; ks < QK; ks++)
#pragma unroll
      for (int e = 0; e < 8; e++) qf[ks][e] = (bf16)((float)qf[ks][e] * cs);
  }
  // Online softmax state: reference max m (log2 units), row sum l, O^T.
  float m = -INFINITY, l = 0.f;
  // (fold) the offset the S blocks in flight carry: m, or 0 while m is -inf
  auto mref = [&]() { return m == -INFINITY ? 0.f : m; };
  auto set_ref = [&](float mn) {  // m = mn (rounded to bf16 under the fold) and its query fragment
    if constexpr (FOLD) {
      m = mn == -INFINITY ? mn : (float)(bf16)mn;
      if (lg == 0) qext[0] = (bf16)(-mref());
    } else {
      m = mn;
    }
  };
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; d++) o[d] = f32x16{0};
  // Register i of block kb holds key k0 + 32kb + 16(i/8) + 8lg + i%8.
  auto mask_rows = [&](f32x16* s, int k0) {
    const int lim = max(-1, min(BKV, qpos - k0)) - 8 * lg;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++)
        if (32 * kb + 16 * (i >> 3) + (i & 7) > lim) s[kb][i] = -INFINITY;
  };
  // Row max of one 32-key block / of both, in log2 units, for S blocks formed
  // with the current reference.
  auto block_max = [&](const f32x16& sb) {
    float xs[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int i = 0; i < 16; i++) xs[i & 3] = fmaxf(xs[i & 3], sb[i]);
    const float mx = halves_max(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])));
    return FOLD ? mx + mref() : mx * cs;
  };
  auto row_max = [&](const f32x16* s) { return fmaxf(block_max(s[0]), block_max(s[1])); };
  // One element e of a P fragment and its part of the row sum (the first
  // four elements of a run start the four partial sums).
  auto pel = [&](float x, float nm, frag& pv, int e, float* ls, bool first) {
    const float p = FOLD ? fast_exp2(x) : fast_exp2(fmaf(x, cs, nm));
    pv[e] = (bf16)p;
    if (first)
      ls[e & 3] = p;
    else
      ls[e & 3] += p;
  };
  auto exps = [&](const f32x16& sb, float nm, frag& p0, frag& p1, float* ls) {
#pragma unroll
    for (int t = 0; t < 8; t++) pel(sb[t], nm, p0, t, ls, t < 4);
#pragma unroll
    for (int t = 0; t < 8; t++) pel(sb[8 + t], nm, p1, t, ls, false);
  };
  // Keeps a phase's softmax results inside the phase: without it the
  // compiler sinks the exponentials next to their later uses, out of the
  // MFMA block they are meant to overlap.
  auto pin = [](frag& p0, frag& p1, float* ls) {
    asm volatile("" : "+v"(p0), "+v"(p1), "+v"(ls[0]), "+v"(ls[1]), "+v"(ls[2]), "+v"(ls[3]));
  };
  auto scale_frag = [](frag& pv, float alpha) {
#pragma unroll
    for (int e = 0; e < 8; e++) pv[e] = (bf16)((float)pv[e] * alpha);
  };
  auto shift = [](f32x16& sb, float by) {
#pragma unroll
    for (int i = 0; i < 16; i++) sb[i] += by;
  };
  // Raise the reference max to mn: rescale O, the row sum and the P blocks
  // already formed (npf of them, in pf) by 2^(m - mn).
  auto raise_ref = [&](float mn, frag* pv, int npf) {
    const float mold = m;
    set_ref(mn);
    const float alpha = mold == -INFINITY ? 1.f : fast_exp2(mold - m);
#pragma unroll
    for (int d = 0; d < DB; d++) o[d] *= alpha;
    l *= alpha;
    for (int q = 0; q < npf; q++) scale_frag(pv[q], alpha);
  };
  auto s_product = [&](int buf, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      s[kb] = FOLD ? M_::mma(kext, qext, f32x16{0}) : f32x16{0};
#pragma unroll
      for (int ks = 0; ks < QK; ks++) s[kb] = M_::mma(kfrag(buf, kb, ks), qf[ks], s[kb]);
    }
  };
  auto pv_product = [&](int buf, const frag* pf, f32x16* o) {
#pragma unroll
    for (int st = 0; st < PK; st++)
#pragma unroll
      for (int d = 0; d < DB; d++) o[d] = M_::mma(vfrag(buf, st, d), pf[st], o[d]);
  };

  const int ntiles = (kfin - kbeg + BKV - 1) / BKV;
  const int kw = min(kend_w, kfin);
  const int ntw = kw > kbeg ? (kw - kbeg + BKV - 1) / BKV : 0;  // tiles this wave computes
  auto needmask = [&](int k0) { return !wfull || k0 + BKV - 1 > qmin_w; };

  frag pf[PK];    // P of the tile whose V^T product comes next
  f32x16 sh;      // that tile's second 32-key block of S (exponentials pending)

  // Prologue: K(0), V^T(0), K(1) in; S(0), its max and first-block P.
  issueK(kbeg, 0);
  issueV(kbeg, 0);
  if (ntiles > 1) issueK(kbeg + BKV, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (ntw > 0) {
    f32x16 s[2];
    s_product(0, s);  // the reference is still -inf: no offset yet
    if (needmask(kbeg)) mask_rows(s, kbeg);
    set_ref(row_max(s));
    if constexpr (FOLD) {
      shift(s[0], -mref());
      shift(s[1], -mref());
    }
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    exps(s[0], m == -INFINITY ? 0.f : -m, pf[0], pf[1], ls);
    l = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    sh = s[1];
  }

  for (int t = 0; t < ntiles; t++) {
    const int P = t & 1;
    const int k0 = kbeg + t * BKV;
    // K(t+1) and V^T(t) have landed; every wave is done with K(t), V^T(t-1).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (k0 + BKV > kend32 && (kend32 % V) != 0) {  // last tile, V^T chunk straddles kend
      fixupV(k0, P);
      __syncthreads();
    }
    // The next tiles' loads: in one burst, or (TSP_ATTN_SPREAD, waves running
    // phase A) one after every second MFMA of phase A, so that the four
    // waves of the workgroup do not all queue on the LDS-DMA path at once.
    const bool spread = TSP_ATTN_SPREAD && t + 1 < ntw;
    const bool doK = t + 2 < ntiles, doV = t + 1 < ntiles;
    if (!spread) {
      if (doK) issueK(k0 + 2 * BKV, P);
      if (doV) issueV(k0 + BKV, 1 - P);
    }
    if (t >= ntw) continue;
    const float nm = m == -INFINITY ? 0.f : -m;
    if (t + 1 < ntw) {
      // phase A: one group per MFMA -- the MFMA, the fragment read PD MFMAs
      // ahead (the last groups read phase B's first V^T fragments) and one
      // element of the pending second block's softmax
      f32x16 s[2];
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
      const int kbuf = 1 - P, vbuf = P;
      constexpr int PD = TSP_PIPE_DIST;  // fragment reads in flight
      frag kq[PD], vq[PD];
      // MFMA i accumulates block i % 2 at k-step i / 2: the two blocks'
      // chains alternate, so no MFMA waits on the one just before it.
#pragma unroll
      for (int i = 0; i < PD; i++) kq[i] = kfrag(kbuf, i & 1, i >> 1);
      if constexpr (FOLD) {
        s[0] = M_::mma(kext, qext, f32x16{0});
        s[1] = M_::mma(kext, qext, f32x16{0});
      } else {
        s[0] = f32x16{0};
        s[1] = f32x16{0};
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const frag f = kq[i % PD];
        if (i + PD < 16)
          kq[i % PD] = kfrag(kbuf, (i + PD) & 1, (i + PD) >> 1);
        else
          vq[i + PD - 16] = vfrag(vbuf, (i + PD - 16) >> 2, (i + PD - 16) & 3);
        s[i & 1] = M_::mma(f, qf[i >> 1], s[i & 1]);
        if (TSP_ATTN_SPREAD && (i & 1)) {
          const int jl = i >> 1;  // the wave's KJ K loads, then its VJ V^T loads
          if (jl < KJ) {
            if (doK) issueK1(k0 + 2 * BKV, P, jl);
          } else if (jl < KJ + VJ && doV) {
            issueV1(k0 + BKV, 1 - P, jl - KJ);
          }
        }
        pel(sh[i], nm, pf[2 + (i >> 3)], i & 7, ls, i < 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin(pf[2], pf[3], ls);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      {
        // The block's exponentials used the running reference m.  A score
        // more than 2^64 above it (or a non-finite sum) is caught on the
        // block sum and repaired here: raise m to the block's max, rescale,
        // redo the block.
        float lsa = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        if (__any(!(lsa <= kSumCap))) {
          const float mold = mref();
          raise_ref(fmaxf(m, block_max(sh)), pf, 2);
          if constexpr (FOLD) {  // sh and S(t+1) carry the old reference
            shift(sh, mold - mref());
            shift(s[0], mold - mref());
            shift(s[1], mold - mref());
          }
          float lr4[4] = {0.f, 0.f, 0.f, 0.f};
          exps(sh, m == -INFINITY ? 0.f : -m, pf[2], pf[3], lr4);
          lsa = (lr4[0] + lr4[1]) + (lr4[2] + lr4[3]);
        }
        l += lsa;
      }
      if (needmask(k0 + BKV)) mask_rows(s, k0 + BKV);
      const float nm2 = m == -INFINITY ? 0.f : -m;
      __builtin_amdgcn_sched_barrier(0);
      // phase B: the V^T(t) products with the first block of S(t+1)'s softmax
      frag pn[2];
      float ls2[4] = {0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const frag f = vq[i % PD];
        if (i + PD < 16) vq[i % PD] = vfrag(vbuf, (i + PD) >> 2, (i + PD) & 3);
        o[i & 3] = M_::mma(f, pf[i >> 2], o[i & 3]);
        pel(s[0][i], nm2, pn[i >> 3], i & 7, ls2, i < 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin(pn[0], pn[1], ls2);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      {
        float lsb = (ls2[0] + ls2[1]) + (ls2[2] + ls2[3]);
        if (__any(!(lsb <= kSumCap))) {
          // O already holds tile t's products (formed with the old m);
          // take the max of both blocks of S(t+1) so its second block passes
          const float mold = mref();
          raise_ref(fmaxf(m, row_max(s)), pf, 0);
          if constexpr (FOLD) {
            shift(s[0], mold - mref());
            shift(s[1], mold - mref());
          }
          float lr4[4] = {0.f, 0.f, 0.f, 0.f};
          exps(s[0], m == -INFINITY ? 0.f : -m, pn[0], pn[1], lr4);
          lsb = (lr4[0] + lr4[1]) + (lr4[2] + lr4[3]);
        }
        l += lsb;
      }
      pf[0] = pn[0];
      pf[1] = pn[1];
      sh = s[1];
    } else {
      // this wave's last tile: the rest of its P, then its V^T product.
      // (The empty asm makes these exponentials differ from phase A's, which
      // the compiler would otherwise compute once above the branch, out of
      // phase A's MFMA block.)
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+v"(sh));
      exps(sh, nm, pf[2], pf[3], ls);
      float lsa = (ls[0] + ls[1]) + (ls[2] + ls[3]);
      if (__any(!(lsa <= kSumCap))) {
        const float mold = mref();
        raise_ref(fmaxf(m, block_max(sh)), pf, 2);
        if constexpr (FOLD) shift(sh, mold - mref());
        float lr4[4] = {0.f, 0.f, 0.f, 0.f};
        exps(sh, m == -INFINITY ? 0.f : -m, pf[2], pf[3], lr4);
        lsa = (lr4[0] + lr4[1]) + (lr4[2] + lr4[3]);
      }
      l += lsa;
      pv_product(P, pf, o);
    }
  }
  const float lt = halves_sum(l);
  const int64_t row = row0 + lr;
  if (nseg == 1) {
    if (qok) {
      const float inv = 1.0f / lt;
      if (a.LSE && lg == 0) a.LSE[((int64_t)head * nb + sb) * a.T + row] = m + log2f(lt);
      T* orow = (T*)a.O + ((int64_t)sb * a.T + row) * a.ldo + head * HD;
#pragma unroll
      for (int d = 0; d < DB; d++)
#pragma unroll
        for (int q = 0; q < 4; q++)
          store4<T>(orow + 32 * d + 8 * q + 4 * lg, o[d][4 * q] * inv, o[d][4 * q + 1] * inv,
                    o[d][4 * q + 2] * inv, o[d][4 * q + 3] * inv);
    }
  } else {
    const int64_t slot = ((((int64_t)head * nb + sb) * a.nqt + qt) * a.maxseg + seg) * BQ + wave * 32 + lr;
    float* op = a.Op + slot * HD;
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int q = 0; q < 4; q++)
        *(float4*)(op + 32 * d + 8 * q + 4 * lg) =
            make_float4(o[d][4 * q], o[d][4 * q + 1], o[d][4 * q + 2], o[d][4 * q + 3]);
    if (lg == 0) {
      a.ML[2 * slot] = m;
      a.ML[2 * slot + 1] = lt;
    }
  }
}

// Merge the partial results of split query tiles:
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  constexpr int DQ = HD / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rid = gid / DQ;
  const int dq = (int)(gid % DQ);
  const int nb = batch_of(a);
  const int64_t BT = (int64_t)nb * a.T;
  const int64_t head = rid / BT, rowg = rid % BT;  // rowg = sb * T + row
  if (head >= a.Hd) return;
  const int64_t sb = rowg / a.T, row = rowg % a.T;
  const int qt = (int)(row / a.bq);
  const int64_t kend = qtile_kend(a.T, qt, a.chunk, a.rank, a.fold, a.bq);
  const int nseg = (int)((kend + a.lseg - 1) / a.lseg);
  if (nseg == 1) return;
  const int64_t base = (((head * nb + sb) * a.nqt + qt) * a.maxseg) * a.bq + (row % a.bq);
  float mx = -INFINITY;
  for (int s = 0; s < nseg; s++) mx = fmaxf(mx, a.ML[2 * (base + s * a.bq)]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nseg; s++) {
    const int64_t slot = base + s * a.bq;
    const float ms = a.ML[2 * slot];
    const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - mx);
    L += w * a.ML[2 * slot + 1];
    const float4 v = *(const float4*)(a.Op + slot * HD + 4 * dq);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = 1.0f / L;
  if (a.LSE && dq == 0) a.LSE[rid] = mx + log2f(L);
  store4<T>((T*)a.O + rowg * a.ldo + head * HD + 4 * dq, acc.x * inv, acc.y * inv, acc.z * inv,
            acc.w * inv);
}

// ---------------------------------------------------------------------------
// Backward of the MLP half (the gradient reading of the oracle's backward
// module: each rank's rows, partial weight gradients).  The products run on
// the projection GEMM; these kernels supply its transposed operands and the
// elementwise and row-wise steps.
// ---------------------------------------------------------------------------

// out[c][r] = in[r][c] for an R x C matrix (row pitches ldi, ldo), through a
// 64 x 64 LDS tile (one padding column against bank conflicts).
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                        int64_t R, int64_t C, int64_t ldi, int64_t ldo) {
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? in[r * ldi + c] : from_f<T>(0.f);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < R) out[c * ldo + r] = tile[tx][i];
  }
}

// The batched, row-padded form: block (x, y, z) moves rows [64 x, 64 x + 64)
// and columns [64 y, 64 y + 64) of matrix z, writing zeros for rows >= R.
template <typename T>
__global__ void __launch_bounds__(256) transpose_pad_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                            int64_t R, int64_t Rp, int64_t C, int64_t ldi,
                                                            int64_t ldo, int64_t zdiv, int64_t s1, int64_t s0) {
  __shared__ T tile[64][65];
  const int64_t z = blockIdx.z;
  const T* src = in + (z / zdiv) * s1 + (z % zdiv) * s0;
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? src[r * ldi + c] : from_f<T>(0.f);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) out[c * ldo + z * Rp + r] = tile[tx][i];
  }
}

// Both forms for bf16 with 16-byte global accesses: a 64 x 64 tile per
// work-group, read as 16-byte chunks of input rows (8 elements) and written as
// 16-byte chunks of output rows gathered from the tile's columns.  Output row
// c, column zs z + r holds input row r, column c of matrix z (at in + (z /
// zdiv) s1 + (z % zdiv) s0); rows R <= r < Rw are written as zeros.  The
// tile's rows are 132 bytes apart, so the eight rows one gather reads at a
// time fall on eight different groups of four banks.  Needs 16-byte aligned
// in and out, and ldi, ldo, s1, s0, zs multiples of 8 elements.
__global__ void __launch_bounds__(256) transpose16_kernel(const bf16* __restrict__ in, bf16* __restrict__ out,
                                                          int64_t R, int64_t Rw, int64_t C, int64_t ldi,
                                                          int64_t ldo, int64_t zdiv, int64_t s1, int64_t s0,
                                                          int64_t zs) {
  constexpr int P = 66;  // tile row pitch in elements (132 bytes)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];
  const int64_t z = blockIdx.z;
  const uint16_t* src = (const uint16_t*)in + (z / zdiv) * s1 + (z % zdiv) * s0;
  uint16_t* dst = (uint16_t*)out + z * zs;
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int q = t + 256 * u, rr = q >> 3, cc = (q & 7) * 8;
    const int64_t r = r0 + rr, c = c0 + cc;
    uint4 v = {0u, 0u, 0u, 0u};
    if (r < R) {
      if (c + 8 <= C) {
        v = *(const uint4*)(src + r * ldi + c);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int k = 0; k < 8 && c + k < C; k++) w[k >> 1] |= (uint32_t)src[r * ldi + c + k] << (16 * (k & 1));
        v = uint4{w[0], w[1], w[2], w[3]};
      }
    }
    uint32_t* row = (uint32_t*)(tile + rr * P + cc);
    row[0] = v.x;
    row[1] = v.y;
    row[2] = v.z;
    row[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int q = t + 256 * u, oc = q >> 3, orr = (q & 7) * 8;
    const int64_t c = c0 + oc, r = r0 + orr;
    if (c >= C || r >= Rw) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
      w[k] = (uint32_t)tile[(orr + 2 * k) * P + oc] | ((uint32_t)tile[(orr + 2 * k + 1) * P + oc] << 16);
    uint16_t* o = dst + c * ldo + r;
    if (r + 8 <= Rw) {
      *(uint4*)o = uint4{w[0], w[1], w[2], w[3]};
    } else {
      for (int k = 0; r + k < Rw; k++) o[k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
    }
  }
}

// SwiGLU backward per element, a = n W1 and b = n W3 given in fp32 side by
// side ([rows][2F]: a in columns [0, F), b in [F, 2F)) and dg = dout W2^T in
// fp32 [rows][F]: da = dg b silu'(a), db = dg silu(a) into
// dab [rows][2F] (da in columns [0, F), db in [F, 2F)), and the forward
// product g = silu(a) b into g [rows][F].
template <typename T>
__global__ void __launch_bounds__(256) swiglu_bwd_kernel(const float* __restrict__ ab,
                                                         const float* __restrict__ dg,
                                                         T* __restrict__ dab, T* __restrict__ g,
                                                         int64_t rows, int64_t F) {
  const int64_t n = rows * F;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / F, c = i - r * F;
    const float av = ab[r * 2 * F + c], bv = ab[r * 2 * F + F + c], gv = dg[i];
    const float sg = 1.0f / (1.0f + expf(-av));
    const float s = av * sg;
    dab[r * 2 * F + c] = from_f<T>(gv * bv * sg * (1.0f + av * (1.0f - sg)));
    dab[r * 2 * F + F + c] = from_f<T>(gv * s);
    g[i] = from_f<T>(s * bv);
  }
}

// RMSNorm backward, one wave per row: with r = (mean(x^2) + eps)^(-1/2) and
// u = dn g, dx = res + r u - x r^3 <u, x> / h (res: the residual gradient
// that passes the norm), and rs[row] = r for the gain's gradient.
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                          const float* __restrict__ dn,
                                                          const T* __restrict__ res, T* __restrict__ dx,
                                                          float* __restrict__ rs, int64_t rows, int h,
                                                          float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + row * h;
  const float* dr = dn + row * h;
  float ss = 0.f, ux = 0.f;
  for (int i = lane; i < h; i += 64) {
    const float xv = to_f(xr[i]);
    ss += xv * xv;
    ux += dr[i] * to_f(g[i]) * xv;
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    ss += __shfl_xor(ss, o);
    ux += __shfl_xor(ux, o);
  }
  const float r = 1.0f / sqrtf(ss / (float)h + eps);
  const float k = r * r * r * ux / (float)h;
  for (int i = lane; i < h; i += 64) {
    const float xv = to_f(xr[i]);
    dx[row * h + i] = from_f<T>(to_f(res[row * h + i]) + r * dr[i] * to_f(g[i]) - xv * k);
  }
  if (lane == 0) rs[row] = r;
}

// Gain gradient, dgain[c] += sum over rows of dn[row][c] x[row][c] rs[row],
// in two passes with a fixed summation order (no atomics, so the result is
// the same on every run).  First pass: partial[b][c] = the sum over rows
// [kGainRows b, kGainRows (b + 1)), one thread per column.
constexpr int kGainRows = 64;
template <typename T>
__global__ void __launch_bounds__(256) gain_grad_kernel(const T* __restrict__ x, const float* __restrict__ dn,
                                                        const float* __restrict__ rs, float* __restrict__ partial,
                                                        int64_t rows, int h) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= h) return;
  const int64_t r0 = (int64_t)blockIdx.y * kGainRows;
  const int64_t r1 = r0 + kGainRows < rows ? r0 + kGainRows : rows;
  float acc = 0.f;
  for (int64_t r = r0; r < r1; r++) acc += dn[r * h + c] * to_f(x[r * h + c]) * rs[r];
  partial[(int64_t)blockIdx.y * h + c] = acc;
}

// Second pass: dgain[c] += the nb partial sums of column c, in block order.
__global__ void __launch_bounds__(256) gain_sum_kernel(const float* __restrict__ partial, float* __restrict__ dgain,
                                                       int64_t nb, int h) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= h) return;
  float s = 0.f;
  for (int64_t b = 0; b < nb; b++) s += partial[b * h + c];
  dgain[c] += s;
}

// ---------------------------------------------------------------------------
// Pieces of the whole layer's backward around the attention core.
// ---------------------------------------------------------------------------

// The rotation's backward: it is orthogonal, so the gradient turns back by
// the opposite angle, i.e. the forward rotation at position -p.  One thread
// per four dims of one row of one head.
__global__ void __launch_bounds__(256) rope_inverse_kernel(float* __restrict__ v, int64_t rows, int heads,
                                                           int hd, int64_t S, int64_t T, int64_t chunk,
                                                           int rank, int fold, double l2c) {
  const int q4 = hd / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)heads * rows * q4) return;
  const int64_t row = (gid / q4) % rows;
  const int e = (int)(gid % q4) * 4;
  const int64_t p = S > 0 ? row % S : zig(row % T, chunk, rank, fold);
  float* pv = v + (gid / q4) * hd + e;
  float4 x = *(float4*)pv;
  float w[4] = {x.x, x.y, x.z, x.w};
  rope_pairs(w, e, -p, l2c);
  *(float4*)pv = make_float4(w[0], w[1], w[2], w[3]);
}

// One thread per four dims of one local row of one (shard, K|V, head): the
// sum over the ranks' partial gradients at that row's position.
__global__ void __launch_bounds__(256) kv_grad_reduce_kernel(KvGradReduceArgs a) {
  const int q4 = a.hd / 4;
  const int64_t BT = a.batch * a.T, BS = a.batch * a.S;
  const int64_t planes = (int64_t)a.fold * 2 * a.hkd;  // (shard, K|V, head) planes
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= planes * BT * q4) return;
  const int e = (int)(gid % q4) * 4;
  const int64_t m = (gid / q4) % BT;
  const int64_t plane = gid / q4 / BT;
  const int64_t b = m / a.T;
  const int64_t src = plane * BS * a.hd + (b * a.S + zig(m - b * a.T, a.chunk, a.rank, a.fold)) * a.hd + e;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < a.fold; q++) {
    const float4 x = *(const float4*)(a.part[q] + src);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  *(float4*)(a.own + plane * BT * a.hd + m * a.hd + e) = acc;
}

// [dQ | dK | dV] of one shard's head group side by side, in the GEMM operand
// dtype: column c < hs is query head c / hd, then ks key and ks value columns.
template <typename T>
__global__ void __launch_bounds__(256) qkv_grad_pack_kernel(const float* __restrict__ dq,
                                                            const float* __restrict__ dk,
                                                            const float* __restrict__ dv, T* __restrict__ out,
                                                            int64_t rows, int hs, int ks, int hd) {
  const int n4 = (hs + 2 * ks) / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= rows * n4) return;
  const int64_t m = gid / n4;
  const int c = (int)(gid % n4) * 4;
  const float* src;
  int cc = c;
  if (c < hs) {
    src = dq;
  } else if (c < hs + ks) {
    src = dk;
    cc = c - hs;
  } else {
    src = dv;
    cc = c - hs - ks;
  }
  const float4 x = *(const float4*)(src + ((int64_t)(cc / hd) * rows + m) * hd + cc % hd);
  store4<T>(out + m * (hs + 2 * ks) + c, x.x, x.y, x.z, x.w);
}

// ---------------------------------------------------------------------------
// Backward of the causal attention core (FlashAttention's recomputation:
// the probabilities are rebuilt from the forward's per-row log-sum-exp, so no
// S x S matrix is stored).  With P the probabilities of a query block
// against a key block, dP = dO V^T, dS = P (dP - rowsum(dO O)):
//   dV = P^T dO,  dK = dS^T Q / sqrt(d),  dQ = dS K / sqrt(d).
// Two kernels, neither with atomics: one owns a key block and walks the query
// blocks that can see it (dK, dV), the other owns a query block and walks
// its keys (dQ, recomputing P and dP).
//
// Every product runs on the 32x32x16 bf16 MFMA.  A lane of its 32x32 result
// holds one column and 16 rows; a lane of its first operand holds one row
// and 8 consecutive k.  So a wave's P (or dS) block, formed with the keys
// (queries in the dQ kernel) as columns, is already the first operand of
// the next product, contracted over the rows, provided the rows come out in
// the right order: the score product reads its first operand's rows through
// the permutation perm_rows, after which register i of a lane holds row
// 16 (i / 8) + 8 (lane / 32) + i % 8.  P and dS never pass through LDS.
//
// Tiles reach LDS by buffer->LDS loads, double-buffered, one barrier per
// block: rows past a tile's valid range read as zero through the buffer's
// range check.  The second operand of a product over the rows of Q, dO or K
// comes from a transposed copy made in HBM before the kernels run, padded
// per sequence to a multiple of 64 rows with zeros, so that those tiles are
// always whole.
// ---------------------------------------------------------------------------
#ifndef TSP_BWD_DIST
#define TSP_BWD_DIST 4  // dK/dV kernel: LDS fragment reads in flight ahead of the MFMAs
#endif
constexpr int kAB = 64;    // rows of a query or key block
constexpr int kBK2 = 128;  // keys per work-group of the dK/dV kernel
constexpr int kBQ2 = 128;  // query rows per work-group of the dQ kernel

// Position of local row i of a rank's zigzag rows (chunks r and 2D-1-r).
__host__ __device__ inline int64_t zz_pos(int64_t i, int64_t C, int r, int D) {
  return i < C ? (int64_t)r * C + i : (2 * (int64_t)D - 1 - r) * C + (i - C);
}

// 64-key blocks that the rows of 128-row query block qb attend to.
__host__ __device__ inline int dq_key_blocks(int64_t qb, int64_t T, int64_t C, int r, int D) {
  const int64_t last = ((qb + 1) * kBQ2 < T ? (qb + 1) * kBQ2 : T) - 1;
  return (int)((zz_pos(last, C, r, D) + kAB) / kAB);
}

void attn_bwd_dq_plan(int64_t T, int64_t chunk, int rank, int fold, int64_t heads, int* seg, int* items) {
  const int64_t nqb = (T + kBQ2 - 1) / kBQ2;
  int64_t total = 0;
  for (int64_t qb = 0; qb < nqb; qb++) total += dq_key_blocks(qb, T, chunk, rank, fold);
  // about two work-groups' worth of work per CU (four measured no faster and
  // doubled the merge), and at least 16 key blocks (1024 keys) per item
  const int64_t sg = std::max<int64_t>(16, (total * heads + 511) / 512);
  int64_t n = 0;
  for (int64_t qb = 0; qb < nqb; qb++) n += (dq_key_blocks(qb, T, chunk, rank, fold) + sg - 1) / sg;
  *seg = (int)sg;
  *items = (int)n;
}

// First local row of rank r whose position reaches p (T if none): positions
// grow with the local row, so the causal test key <= pos(row) is
// row >= first_row_at(key).
__device__ inline int64_t first_row_at(int64_t p, int64_t C, int r, int D, int64_t T) {
  const int64_t ca = (int64_t)r * C, cb = (2 * (int64_t)D - 1 - r) * C;
  return p <= ca ? 0 : p < ca + C ? p - ca : p <= cb ? C : p < cb + C ? C + p - cb : T;
}

// Row read by first-operand lane row rho of a score product: swaps the middle
// two groups of four in every 16 (0-3, 8-11, 4-7, 12-15), so that result
// register i of a lane holds row 16 (i / 8) + 8 (lane / 32) + i % 8.
__device__ inline int perm_rows(int rho) { return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

// 4 bytes per lane from buffer offset voff into LDS at lds + 4*lane.
__device__ inline void buffer_to_lds4(brsrc r, void* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, voff, 0, 0, 0);
#endif
}

// A tile of R rows of RB bytes (row r at byte r * ld of the buffer) into LDS
// rows of RB bytes, 16-byte chunks XOR-swizzled with swz<RB / 16>: each wave
// instruction moves 1 KB, spread over the work-group's NW waves.
template <int R, int RB, int NW>
__device__ inline void dma_tile(brsrc src, uint32_t ld, char* lds, int w, int lane) {
  constexpr int NCH = RB / 16, RPI = 1024 / RB, NI = R * RB / 1024;
  static_assert(NI % NW == 0, "the tile must split evenly over the waves");
#pragma unroll
  for (int j = 0; j < NI / NW; j++) {
    const int ins = w + NW * j;
    const int row = ins * RPI + lane / NCH;
    buffer_to_lds16(src, lds + ins * 1024, (uint32_t)row * ld + (uint32_t)swz<NCH>(lane % NCH, row) * 16, 0);
  }
}

// The 16 bytes at logical chunk c of row r of such a tile.
template <int RB>
__device__ inline bf16x8 lds_chunk(const char* tile, int r, int c) {
  return *(const bf16x8*)(tile + r * RB + swz<RB / 16>(c, r) * 16);
}

// Dl = rowsum(dO * O) per head and row; one wave per (head, row).
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_delta_kernel(AttnBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t BT = (int64_t)a.batch * a.T;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)a.Hd * BT) return;
  const int64_t t = item / BT, rowg = item % BT;
  const bf16* o = (const bf16*)a.O + rowg * a.ldo_fwd + t * HD;
  const bf16* g = (const bf16*)a.dO + rowg * a.ldo + t * HD;
  float s = 0.f;
  for (int e = lane; e < HD; e += 64) s += (float)o[e] * (float)g[e];
  for (int off = 32; off; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) a.Dl[item] = s;
}

// One work-group per (128-key block, K/V head, sequence): dK and dV of those
// keys, summed over the head's query heads and every query row of the rank
// that attends to them.  Four waves, one per SIMD: wave w owns keys 32 w..
// of the block, with K and V in registers, and walks the 64-row query blocks
// that reach them as two independent 32-row halves, so that the softmax of
// one half can overlap the other half's MFMAs within the wave.  Per block:
// Q, dO (rows) and Q^T, dO^T (from Qt, dOt [HD][Hd][B][Tp]), with the rows'
// LSE and Dl.
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int RB = HD * 2;        // bytes of a row of a row-major tile
  constexpr int TB = kAB * HD * 2;  // bytes of a 64 x HD tile, either layout
  constexpr int NKB = HD / 32;      // 32-wide blocks of the head dimension
  constexpr int KS = HD / 16;       // k steps of a product over the head dimension
  constexpr int NW = 4;
  static_assert(2 * kBK2 * RB <= 8 * TB, "K and V staging must fit in the loop's space");
  __shared__ __attribute__((aligned(1024))) char sm[2 * 4 * TB];  // two buffers of [Q | dO | Q^T | dO^T]
  __shared__ float lsd[2][2][kAB];                                // per buffer: the rows' LSE, Dl
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t k0 = (int64_t)blockIdx.x * kBK2;
  const int hk = blockIdx.y, b = blockIdx.z;
  const int64_t BS = (int64_t)a.batch * a.S;
  const int nkeys = (int)std::min<int64_t>(kBK2, a.S - k0);
  bf16x8 kf[KS], vf[KS];  // second operands of S and dP: the wave's 32 keys of K and V
  {
    const bf16* kb = (const bf16*)a.K + ((int64_t)hk * BS + (int64_t)b * a.S + k0) * HD;
    const bf16* vb = (const bf16*)a.Vr + ((int64_t)b * a.S + k0) * a.Hkd * HD + (int64_t)hk * HD;
    const uint32_t ldv = (uint32_t)a.Hkd * RB;
    dma_tile<kBK2, RB, NW>(make_rsrc(kb, (uint64_t)nkeys * RB), RB, sm, w, lane);
    dma_tile<kBK2, RB, NW>(make_rsrc(vb, (uint64_t)(nkeys - 1) * ldv + RB), ldv, sm + kBK2 * RB, w, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int r = 32 * w + l32;
#pragma unroll
    for (int k = 0; k < KS; k++) {
      kf[k] = lds_chunk<RB>(sm, r, 2 * k + h);
      vf[k] = lds_chunk<RB>(sm + kBK2 * RB, r, 2 * k + h);
    }
    __syncthreads();  // every wave holds its fragments before the loop's loads reuse the space
  }
  const int64_t qs = first_row_at(k0, a.chunk, a.rank, a.fold, a.T) / kAB * kAB;
  const int nqb = (int)((a.T - qs + kAB - 1) / kAB);
  const int total = a.grp * nqb;  // (query head, query block) pairs, head-major
  const uint32_t ldt = (uint32_t)((int64_t)a.Hd * a.batch * a.Tp * 2);  // bytes per row of Qt, dOt
  const uint32_t ldo = (uint32_t)a.ldo * 2;
  auto issue = [&](int it, int buf) {
    const int64_t t = (int64_t)hk * a.grp + it / nqb, q0 = qs + (int64_t)kAB * (it % nqb);
    const int nq = (int)std::min<int64_t>(kAB, a.T - q0);
    char* base = sm + buf * 4 * TB;
    const int64_t row0 = (t * a.batch + b) * a.T + q0;
    dma_tile<kAB, RB, NW>(make_rsrc((const bf16*)a.Q + row0 * HD, (uint64_t)nq * RB), RB, base, w, lane);
    dma_tile<kAB, RB, NW>(make_rsrc((const bf16*)a.dO + ((int64_t)b * a.T + q0) * a.ldo + t * HD,
                                    (uint64_t)(nq - 1) * ldo + RB),
                          ldo, base + TB, w, lane);
    const int64_t col = (t * a.batch + b) * a.Tp + q0;
    const uint64_t tbytes = (uint64_t)(HD - 1) * ldt + 128;
    dma_tile<HD, 128, NW>(make_rsrc((const bf16*)a.Qt + col, tbytes), ldt, base + 2 * TB, w, lane);
    dma_tile<HD, 128, NW>(make_rsrc((const bf16*)a.dOt + col, tbytes), ldt, base + 3 * TB, w, lane);
    if (w == 0) {
      buffer_to_lds4(make_rsrc(a.LSE + row0, (uint64_t)nq * 4), lsd[buf][0], (uint32_t)lane * 4);
      buffer_to_lds4(make_rsrc(a.Dl + row0, (uint64_t)nq * 4), lsd[buf][1], (uint32_t)lane * 4);
    }
  };
  f32x16 dk[NKB], dv[NKB];
#pragma unroll
  for (int u = 0; u < NKB; u++)
#pragma unroll
    for (int i = 0; i < 16; i++) dk[u][i] = dv[u][i] = 0.f;
  // the lane's key (its column of S) is seen by local rows [qk, T)
  const int64_t qk = first_row_at(k0 + 32 * w + l32, a.chunk, a.rank, a.fold, a.T);
  // rows from here on see all of the wave's keys (first_row_at grows with the key)
  const int64_t qk_all = first_row_at(k0 + 32 * w + 31, a.chunk, a.rank, a.fold, a.T);
  const int qr = perm_rows(l32);  // the row of each 32-row half the lane feeds into S and dP
  if (total > 0) issue(0, 0);
  for (int it = 0; it < total; it++) {
    const int buf = it & 1;
    const int64_t q0 = qs + (int64_t)kAB * (it % nqb);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // this block's tiles have landed, and no wave still reads the other buffer
    if (it + 1 < total) issue(it + 1, buf ^ 1);
    const char* Qs = sm + buf * 4 * TB;
    const char* dOs = Qs + TB;
    const char* Qt = Qs + 2 * TB;
    const char* dOt = Qs + 3 * TB;
    // P and dS as first operands: register i of half qh holds block row
    // 32 qh + 8 h + 16 (i / 8) + i % 8, kept when that row is in [lo, hi)
    const int lo = (int)std::min<int64_t>(std::max<int64_t>(qk - q0, 0), kAB) - 8 * h;
    const int hi = (int)std::min<int64_t>(a.T - q0, kAB) - 8 * h;
    // the rows' LSE and Dl, 16 of each per half
    float4 lr[2][4], dr[2][4];
#pragma unroll
    for (int qh = 0; qh < 2; qh++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int m = 32 * qh + 16 * (j >> 1) + 8 * h + 4 * (j & 1);
        lr[qh][j] = *(const float4*)&lsd[buf][0][m];
        dr[qh][j] = *(const float4*)&lsd[buf][1][m];
      }
    // MFMA steps: S and dP of half 0 (2 KS steps), of half 1 (2 KS, with
    // half 0's softmax), dV and dK of half 0 (4 NKB, with half 1's softmax),
    // of half 1 (4 NKB).  Step i reads the operand of step i + PD from LDS.
    // Alternate steps feed different accumulators, so no MFMA waits on the
    // one before.
    // A block whose 64 rows all lie in [qk_all, T) needs no mask.  The
    // softmax below forms P and dS unmasked; on the other blocks each half's
    // entries outside [lo, hi) are zeroed in the packed bf16 operands just
    // before the dV / dK products read them (they may hold inf or NaN for
    // rows past T, which the select drops).
    const bool full = q0 >= qk_all && q0 + kAB <= a.T;
    constexpr int PD = TSP_BWD_DIST, NA = 2 * KS, NB = 4 * NKB, NS = 2 * (NA + NB);
    constexpr int EA = 16 / NA, EB = 16 / NB;  // softmax elements per step
    static_assert(16 % NA == 0 && 16 % NB == 0, "softmax elements must spread evenly over the steps");
    auto frag_at = [&](int i) -> bf16x8 {
      if (i < 2 * NA) {
        const int qh = i / NA, k = (i % NA) >> 1;
        return lds_chunk<RB>((i & 1) ? dOs : Qs, 32 * qh + qr, 2 * k + h);
      }
      const int qh = (i - 2 * NA) / NB, j = (i - 2 * NA) % NB, s2 = j / (2 * NKB), u = (j % (2 * NKB)) >> 1;
      return lds_chunk<128>((j & 1) ? Qt : dOt, 32 * u + l32, 4 * qh + 2 * s2 + h);
    };
    // (each half's first S and dP products start from a zero accumulator)
    f32x16 s[2], dp[2];
    bf16x8 pa[2][2], da[2][2];
    auto soft = [&](int qh, int i) {  // softmax element i of half qh
      const float4 l4 = lr[qh][i >> 2], d4 = dr[qh][i >> 2];
      const int e = i & 3;
      const float lv = e == 0 ? l4.x : e == 1 ? l4.y : e == 2 ? l4.z : l4.w;
      const float dl = e == 0 ? d4.x : e == 1 ? d4.y : e == 2 ? d4.z : d4.w;
      const int c = 32 * qh + 16 * (i >> 3) + (i & 7);
      (void)c;
      const float pr = fast_exp2(s[qh][i] * a.scale_log2 - lv);
      pa[qh][i >> 3][i & 7] = (bf16)pr;
      da[qh][i >> 3][i & 7] = (bf16)(pr * (dp[qh][i] - dl));
    };
    auto mask_half = [&](int qh) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int c = 32 * qh + 16 * (i >> 3) + (i & 7);
        const bool keep = c >= lo && c < hi;
        pa[qh][i >> 3][i & 7] = keep ? pa[qh][i >> 3][i & 7] : (bf16)0.f;
        da[qh][i >> 3][i & 7] = keep ? da[qh][i >> 3][i & 7] : (bf16)0.f;
      }
    };
    bf16x8 ring[PD];
#pragma unroll
    for (int i = 0; i < PD; i++) ring[i] = frag_at(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qh = 0; qh < 2; qh++) {
#pragma unroll
      for (int j = 0; j < NA; j++) {
        const int i = NA * qh + j;
        const bf16x8 f = ring[i % PD];
        ring[i % PD] = frag_at(i + PD);
        if (j & 1)
          dp[qh] = MF<bf16>::mma(f, vf[j >> 1], j < 2 ? f32x16{0} : dp[qh]);
        else
          s[qh] = MF<bf16>::mma(f, kf[j >> 1], j < 2 ? f32x16{0} : s[qh]);
        if (qh == 1)
#pragma unroll
          for (int e = 0; e < EA; e++) soft(0, EA * j + e);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int qh = 0; qh < 2; qh++) {
      if (!full) {  // this half's P and dS are complete: drop the rows its keys do not see
        mask_half(qh);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < NB; j++) {
        const int i = 2 * NA + NB * qh + j, s2 = j / (2 * NKB), u = (j % (2 * NKB)) >> 1;
        const bf16x8 f = ring[i % PD];
        if (i + PD < NS) ring[i % PD] = frag_at(i + PD);
        if (j & 1)
          dk[u] = MF<bf16>::mma(da[qh][s2], f, dk[u]);
        else
          dv[u] = MF<bf16>::mma(pa[qh][s2], f, dv[u]);
        if (qh == 0)
#pragma unroll
          for (int e = 0; e < EB; e++) soft(1, EB * j + e);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NKB; u++) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int64_t kk = k0 + 32 * w + 8 * (i >> 2) + 4 * h + (i & 3);
      if (kk < a.S) {
        const int64_t off = ((int64_t)hk * BS + (int64_t)b * a.S + kk) * HD + 32 * u + l32;
        a.dK[off] = dk[u][i] * a.scale;
        a.dV[off] = dv[u][i];
      }
    }
  }
}

// One work-group per (128-row query block, query head, sequence): dQ of
// those rows over every key they attend to.  Eight waves: wave (qh, kh) owns
// queries 32 qh.. of the block, with Q and dO in registers, and keys 32 kh..
// of each 64-key block; the scores are formed transposed (keys by rows), so
// dS is the first operand of dQ = dS K.  The two key halves are added once
// at the end.  Per key block: K and V (rows) and K^T (from Kt [HD][Hkd][B][Sp]).
template <int HD>
__global__ void __launch_bounds__(512) attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int RB = HD * 2;
  constexpr int TB = kAB * HD * 2;
  constexpr int NKB = HD / 32;
  constexpr int KS = HD / 16;
  static_assert(2 * kBQ2 * RB <= 6 * TB, "Q and dO staging must fit in the loop's space");
  __shared__ __attribute__((aligned(1024))) char sm[2 * 3 * TB];  // two buffers of [K | V | K^T]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int qh = w >> 1, kh = w & 1;
  // item -> (query block, key segment): blocks in order, each split into
  // ceil(nkb / dq_seg) segments of equal length
  int64_t qb = 0;
  int seg = blockIdx.x, nkbq = dq_key_blocks(0, a.T, a.chunk, a.rank, a.fold);
  for (int ns = (nkbq + a.dq_seg - 1) / a.dq_seg; seg >= ns; ns = (nkbq + a.dq_seg - 1) / a.dq_seg) {
    seg -= ns;
    nkbq = dq_key_blocks(++qb, a.T, a.chunk, a.rank, a.fold);
  }
  const int nseg = (nkbq + a.dq_seg - 1) / a.dq_seg, slen = (nkbq + nseg - 1) / nseg;
  const int kb_begin = seg * slen, kb_end = std::min(nkbq, kb_begin + slen);
  const int64_t q0 = qb * kBQ2;
  const int64_t t = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t hk = t / a.grp;
  const int64_t BS = (int64_t)a.batch * a.S;
  const int nq = (int)std::min<int64_t>(kBQ2, a.T - q0);
  const uint32_t ldo = (uint32_t)a.ldo * 2;
  bf16x8 qf[KS], of[KS];  // second operands of S^T and dP^T: the wave's 32 queries of Q and dO
  {
    dma_tile<kBQ2, RB, 8>(make_rsrc((const bf16*)a.Q + ((t * a.batch + b) * a.T + q0) * HD, (uint64_t)nq * RB),
                          RB, sm, w, lane);
    dma_tile<kBQ2, RB, 8>(make_rsrc((const bf16*)a.dO + ((int64_t)b * a.T + q0) * a.ldo + t * HD,
                                    (uint64_t)(nq - 1) * ldo + RB),
                          ldo, sm + kBQ2 * RB, w, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int r = 32 * qh + l32;
#pragma unroll
    for (int k = 0; k < KS; k++) {
      qf[k] = lds_chunk<RB>(sm, r, 2 * k + h);
      of[k] = lds_chunk<RB>(sm + kBQ2 * RB, r, 2 * k + h);
    }
    __syncthreads();
  }
  const int mq = 32 * qh + l32;  // the lane's query (its column of S^T)
  const bool qok = mq < nq;
  const int64_t qpos = qok ? zz_pos(q0 + mq, a.chunk, a.rank, a.fold) : -1;
  const int64_t rr = (t * a.batch + b) * a.T + q0 + mq;
  const float lq = qok ? a.LSE[rr] : 0.f, dlq = qok ? a.Dl[rr] : 0.f;
  const uint32_t ldk = (uint32_t)((int64_t)a.Hkd * a.batch * a.Sp * 2);  // bytes per row of Kt
  const uint32_t ldv = (uint32_t)a.Hkd * RB;
  auto issue = [&](int64_t kb0, int buf) {
    const int nk = (int)std::min<int64_t>(kAB, a.S - kb0);
    char* base = sm + buf * 3 * TB;
    dma_tile<kAB, RB, 8>(make_rsrc((const bf16*)a.K + (hk * BS + (int64_t)b * a.S + kb0) * HD, (uint64_t)nk * RB),
                         RB, base, w, lane);
    dma_tile<kAB, RB, 8>(make_rsrc((const bf16*)a.Vr + ((int64_t)b * a.S + kb0) * a.Hkd * HD + hk * HD,
                                   (uint64_t)(nk - 1) * ldv + RB),
                         ldv, base + TB, w, lane);
    dma_tile<HD, 128, 8>(make_rsrc((const bf16*)a.Kt + (hk * a.batch + b) * a.Sp + kb0,
                                   (uint64_t)(HD - 1) * ldk + 128),
                         ldk, base + 2 * TB, w, lane);
  };
  f32x16 dq[NKB];
#pragma unroll
  for (int u = 0; u < NKB; u++)
#pragma unroll
    for (int i = 0; i < 16; i++) dq[u][i] = 0.f;
  const int kr = 32 * kh + perm_rows(l32);  // the key row the lane feeds into S^T and dP^T
  // the wave's smallest query position (positions grow with the row), or -1
  // when some of its 32 rows lie past the block's last row
  const int64_t qpos_w = 32 * qh + 31 < nq ? zz_pos(q0 + 32 * qh, a.chunk, a.rank, a.fold) : -1;
  if (kb_begin < kb_end) issue((int64_t)kb_begin * kAB, 0);
  for (int kb = kb_begin; kb < kb_end; kb++) {
    const int buf = (kb - kb_begin) & 1;
    const int64_t k0 = (int64_t)kb * kAB;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // this block's tiles have landed, and no wave still reads the other buffer
    if (kb + 1 < kb_end) issue(k0 + kAB, buf ^ 1);
    const char* Ks = sm + buf * 3 * TB;
    const char* Vs = Ks + TB;
    const char* Kt = Ks + 2 * TB;
    f32x16 s, dp;  // (the first products start from a zero accumulator)
#pragma unroll
    for (int k = 0; k < KS; k++) {
      s = MF<bf16>::mma(lds_chunk<RB>(Ks, kr, 2 * k + h), qf[k], k == 0 ? f32x16{0} : s);
      dp = MF<bf16>::mma(lds_chunk<RB>(Vs, kr, 2 * k + h), of[k], k == 0 ? f32x16{0} : dp);
    }
    // dS as the first operand over the wave's 32 keys: register i holds key
    // k0 + 32 kh + 8 h + 16 (i / 8) + i % 8, kept while that key <= qpos.
    // Formed unmasked; when some of the wave's rows do not see all its keys
    // the entries past them are zeroed afterwards (they may hold inf or NaN,
    // which the select drops).
    bf16x8 da[2];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float e = fast_exp2(s[i] * a.scale_log2 - lq);
      da[i >> 3][i & 7] = (bf16)(e * (dp[i] - dlq));
    }
    if (!(qpos_w >= k0 + 32 * kh + 31)) {
      const int lim = (int)std::max<int64_t>(std::min<int64_t>(qpos - k0 - 32 * kh - 8 * h, kAB), -1);
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int c = 16 * (i >> 3) + (i & 7);
        da[i >> 3][i & 7] = c <= lim ? da[i >> 3][i & 7] : (bf16)0.f;
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; s2++) {
      const int c = 4 * kh + 2 * s2 + h;  // the 8 keys' chunk in the K^T tile
#pragma unroll
      for (int u = 0; u < NKB; u++) dq[u] = MF<bf16>::mma(da[s2], lds_chunk<128>(Kt, 32 * u + l32, c), dq[u]);
    }
  }
  __syncthreads();
  float* red = (float*)sm;  // [qh][NKB][16][64]
  if (kh == 1) {
#pragma unroll
    for (int u = 0; u < NKB; u++)
#pragma unroll
      for (int i = 0; i < 16; i++) red[((qh * NKB + u) * 16 + i) * 64 + lane] = dq[u][i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int u = 0; u < NKB; u++) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int m = 32 * qh + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < nq)
          a.dQp[(((t * a.batch + b) * a.dq_items + blockIdx.x) * kBQ2 + m) * HD + 32 * u + l32] =
              dq[u][i] + red[((qh * NKB + u) * 16 + i) * 64 + lane];
      }
    }
  }
}

// dQ of each row: the sum, in segment order, of its query block's item
// partials, times 1/sqrt(d).  One work-group per (128-row query block, head
// and sequence); each thread finds the block's items once.
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_dq_merge_kernel(AttnBwdArgs a) {
  const int64_t qb = blockIdx.x, tb = blockIdx.y;
  int first = 0;
  for (int64_t q = 0; q < qb; q++) first += (dq_key_blocks(q, a.T, a.chunk, a.rank, a.fold) + a.dq_seg - 1) / a.dq_seg;
  const int nseg = (dq_key_blocks(qb, a.T, a.chunk, a.rank, a.fold) + a.dq_seg - 1) / a.dq_seg;
  const int nq = (int)std::min<int64_t>(kBQ2, a.T - qb * kBQ2);
  const float* src = a.dQp + (tb * a.dq_items + first) * kBQ2 * HD;
  for (int e = threadIdx.x; e < nq * (HD / 4); e += 256) {
    const int m = e / (HD / 4), c = 4 * (e % (HD / 4));
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sg = 0; sg < nseg; sg++) {
      const float4 v = *(const float4*)(src + ((int64_t)sg * kBQ2 + m) * HD + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *(float4*)(a.dQ + (tb * a.T + qb * kBQ2 + m) * HD + c) =
        float4{acc.x * a.scale, acc.y * a.scale, acc.z * a.scale, acc.w * a.scale};
  }
}

// ---------------------------------------------------------------------------
// Small helpers for the shard stream's debug modes.
// ---------------------------------------------------------------------------
__global__ void fill32_kernel(uint32_t* p, uint32_t pat, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = pat;
}

__global__ void spin_kernel(uint64_t ticks) {
  if (threadIdx.x == 0) {
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
  }
}

// Clock probe: one lane records n pairs (wall-clock ticks, shader-clock
// cycles), one every `interval` wall-clock ticks.  The shader clock
// (s_memtime) runs at the graphics clock the chip actually sustains; the wall
// clock (s_memrealtime) at a fixed rate, so the ratio of their increments is
// the effective clock while other kernels run beside the probe.  Every wait
// ends: the wall clock only moves forward, and the launcher bounds n*interval.
__global__ void clock_probe_kernel(uint64_t* __restrict__ out, int n, uint64_t interval) {
  if (threadIdx.x != 0) return;
  uint64_t next = wall_clock64();
  for (int i = 0; i < n; i++) {
    uint64_t rt = wall_clock64();
    while (rt < next) {
      __builtin_amdgcn_s_sleep(2);
      rt = wall_clock64();
    }
    const uint64_t ck = clock64();
    out[2 * i] = rt;
    out[2 * i + 1] = ck;
    next = rt + interval;
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
// Split length for the attention work items: the candidate whose simulated
// schedule (items dispatched in order onto 256 CUs, each taking the first
// free one; cost = keys + a fixed per-item overhead + a merge cost per split
// item) finishes first.  Cached per shape.
bool attn_wide(Dtype dt, int hd) { return TSP_ATTN_WIDE && dt == BF16 && hd == 128; }

AttnPlan attn_plan(int64_t T, int64_t S, int64_t chunk, int rank, int fold, int Hd, bool wide) {
  AttnPlan p{};
  p.bq = wide ? kBQW : kBQ;
  p.nqt = (int)((T + p.bq - 1) / p.bq);
  if (T <= 0) return p;
  struct Key { int64_t T, S, C; int r, D, Hd; bool wide; };
  struct Entry { Key k; AttnPlan p; };
  static thread_local std::vector<Entry> cache;
  for (const Entry& e : cache)
    if (e.k.T == T && e.k.S == S && e.k.C == chunk && e.k.r == rank && e.k.D == fold && e.k.Hd == Hd &&
        e.k.wide == wide)
      return e.p;
  std::vector<int64_t> kend(p.nqt);
  int64_t kmax = 0;
  for (int qt = 0; qt < p.nqt; qt++) {
    kend[qt] = qtile_kend(T, qt, chunk, rank, fold, p.bq);
    kmax = std::max(kmax, kend[qt]);
  }
  const int64_t kmax64 = (kmax + 63) / 64 * 64;
  const int kCU = wide ? 256 : 256 * (kQB == 1 ? TSP_ATTN128_WAVES : 1);  // concurrent workgroups
  const double overhead = 3 * kBKV, merge = 2 * kBKV;  // in key units
  double best = 1e300;
  int64_t best_l = kmax64;
  std::vector<double> cu(kCU);
  for (int64_t lseg = 1024; ; lseg += 256) {
    if (lseg > kmax64) lseg = kmax64;
    std::fill(cu.begin(), cu.end(), 0.0);
    // dispatch order (as decode_item): segment-major, heaviest query tiles
    // first within a segment, heads innermost
    int64_t items = 0;
    const int maxs = (int)((kmax + lseg - 1) / lseg);
    for (int sg = 0; sg < maxs; sg++) {
      for (int qt = p.nqt - 1; qt >= 0; --qt) {
        const int ns = (int)((kend[qt] + lseg - 1) / lseg);
        if (sg >= ns) continue;
        const double keys = (double)std::min(lseg, kend[qt] - sg * lseg);
        const double cost = keys + overhead + (ns > 1 ? merge : 0.0);
        for (int h = 0; h < Hd; h++) {
          auto it = std::min_element(cu.begin(), cu.end());
          *it += cost;
          items++;
        }
      }
    }
    const double span = *std::max_element(cu.begin(), cu.end());
    if (span < best * 0.999) {
      best = span;
      best_l = lseg;
    }
    if (lseg >= kmax64) break;
  }
  p.lseg = (int)best_l;
  p.maxseg = 1;
  p.nitems = 0;
  for (int qt = 0; qt < p.nqt; qt++) {
    const int ns = (int)((kend[qt] + best_l - 1) / best_l);
    p.maxseg = std::max(p.maxseg, ns);
    p.nitems += ns;
  }
  p.split = p.maxseg > 1;
  cache.push_back({{T, S, chunk, rank, fold, Hd, wide}, p});
  return p;
}

hipError_t launch_rmsnorm(Dtype dt, const void* x, const void* g, void* y, int64_t rows, int h,
                          float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (dt == BF16)
    rmsnorm_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, rows, h, eps);
  else
    rmsnorm_kernel<float><<<grid, 256, 0, s>>>((const float*)x, (const float*)g, (float*)y, rows, h,
                                               eps);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int EPI, int NW = 4, int WGM = 2>
static void gemm_go(const GemmArgs& a, bool vec, hipStream_t s) {
  const int nt = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (vec)
    gemm_kernel<T, BM, BN, EPI, true, NW, WGM><<<nt, NW * 64, 0, s>>>(a);
  else
    gemm_kernel<T, BM, BN, EPI, false, NW, WGM><<<nt, NW * 64, 0, s>>>(a);
}

// Tile choice.  With every CU holding work the tile shapes reach about the
// same MFMA rate per CU; what differs is how a shape's tile count fills 256
// CUs (4-wave tiles run two workgroups per CU, and a CU with only one of them
// runs it well below that rate).  Measured on the layer's projections at
// 2048, 8192 and 16384 local tokens of the 7B shape:
//  * fp32-accumulator GEMMs (O, W2): 256x256 (ping-pong) when that makes at
//    least one full round of 256 tiles; else 128x128 (4 waves);
//  * QKV: 128x192 when 256x192 needs more than one round; else 4-wave
//    128x192 tiles (two per CU) when they fill at least 3/4 of the 512
//    slots (8192 tokens), else 4-wave 128x128 when they fill half (the
//    narrow N of grouped K/V), else 4-wave 64x64 (2048 tokens);
//  * W1/W3 (two B operands), up to two rounds of 128x192: 4-wave 128x96
//    tiles when they fill 3/4 of the 512 slots (two shards per launch at
//    2048 tokens: 0.104 ms against 0.123 for 128x64), else 4-wave 128x64
//    (one shard at 2048 tokens); beyond that the estimate.
// The estimate: rounds of 256 tiles x tile area / relative efficiency.
#ifndef TSP_ACC_SMALL
#define TSP_ACC_SMALL 1
#endif
//
// The bf16 W1/W3 tile for M x N, named by its width: 96 (4-wave 128x96), 64
// (4-wave 128x64), 128 (8-wave 256x128) or 192 (8-wave 128x192).
static int swiglu_tile_n(int M, int N) {
  auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(128, 192) <= 512)  // 4-wave tiles, two per CU: 128x96 when they fill 3/4 of the 512 slots
    return tiles(128, 96) >= 384 ? 96 : 64;
  // rounds of 256 tiles x tile area / relative efficiency (128x192: 0.8)
  const double t128 = (double)((tiles(256, 128) + 255) / 256) * 256 * 128;
  const double t192 = (double)((tiles(128, 192) + 255) / 256) * 128 * 192 / 0.8;
  return t192 < t128 * 0.999 ? 192 : 128;
}

template <int EPI>
static void gemm_bf16(const GemmArgs& a, bool vec, hipStream_t s) {
  auto tiles = [&](int bm, int bn) {
    return (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  };
  if constexpr (EPI == EPI_SWIGLU) {
    switch (swiglu_tile_n(a.M, a.N)) {
      case 96: gemm_go<bf16, 128, 96, EPI, 4, 4>(a, vec, s); break;
      case 64: gemm_go<bf16, 128, 64, EPI, 4, 2>(a, vec, s); break;
      case 128: gemm_go<bf16, 256, 128, EPI, 8>(a, vec, s); break;
      default: gemm_go<bf16, 128, 192, EPI, 8, 4>(a, vec, s); break;
    }
  } else if constexpr (EPI == EPI_ACC || EPI == EPI_RESID || EPI == EPI_STORE) {
    if (tiles(256, 256) >= 256) gemm_go<bf16, 256, 256, EPI, 8>(a, vec, s);
    else if (tiles(128, 128) >= 256 || !TSP_ACC_SMALL) gemm_go<bf16, 128, 128, EPI, 4, 2>(a, vec, s);
    else gemm_go<bf16, 64, 64, EPI, 4, 2>(a, vec, s);  // small outputs (a shard's dW_O): fill the CUs
  } else {
    if (tiles(256, 192) > 256 && a.hd % 32 == 0) {
      // more than one round of tiles: 256 x 256 (the head dim a multiple of
      // 32, so every 32-column block of the epilogue lies in one head)
      gemm_go<bf16, 256, 256, EPI, 8>(a, vec, s);
    } else if (tiles(256, 192) > 256) {
      gemm_go<bf16, 128, 192, EPI, 8, 4>(a, vec, s);
    } else if (tiles(128, 192) >= 384) {
      // one round of 4-wave 128x192 tiles, two per CU, filling >= 3/4 of them
      gemm_go<bf16, 128, 192, EPI, 4, 2>(a, vec, s);
    } else if (tiles(128, 128) >= 256) {
      gemm_go<bf16, 128, 128, EPI>(a, vec, s);
    } else {
      // few rows (2048 tokens): 4-wave 64x64 tiles, three or more per CU
      gemm_go<bf16, 64, 64, EPI>(a, vec, s);
    }
  }
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

hipError_t launch_gemm(Dtype dt, Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.n_split != 0) {
    if (epi != EPI_SWIGLU || a.n_split < 0 || a.n_split >= a.N || !a.B_2 || !a.B3_2) return hipErrorInvalidValue;
    // one launch when the split falls on a tile boundary, else the two
    // blocks as two launches
    const int bn = dt == BF16 ? swiglu_tile_n(a.M, a.N) : 64;
    if (a.n_split % bn != 0) {
      GemmArgs p = a;
      p.n_split = 0;
      p.N = a.n_split;
      hipError_t e = launch_gemm(dt, epi, p, s);
      if (e != hipSuccess) return e;
      p.B = a.B_2;
      p.B3 = a.B3_2;
      p.N = a.N - a.n_split;
      p.C = (char*)a.C + (size_t)a.n_split * (dt == BF16 ? 2 : 4);
      return launch_gemm(dt, epi, p, s);
    }
  }
  const int V = dt == BF16 ? 8 : 4;
  const bool vec = a.K % V == 0 && a.lda % V == 0 && a.ldb % V == 0 && aligned16(a.A) &&
                   aligned16(a.B) && (a.B3 == nullptr || aligned16(a.B3)) &&
                   (a.n_split == 0 || (aligned16(a.B_2) && aligned16(a.B3_2)));
  if (dt == BF16) {
    switch (epi) {
      case EPI_ACC: gemm_bf16<EPI_ACC>(a, vec, s); break;
      case EPI_RESID: gemm_bf16<EPI_RESID>(a, vec, s); break;
      case EPI_QKV:
        if (a.rope_l2 > 0.0)
          gemm_bf16<EPI_QKV_ROPE>(a, vec, s);
        else
          gemm_bf16<EPI_QKV>(a, vec, s);
        break;
      case EPI_QKV_ROPE: gemm_bf16<EPI_QKV_ROPE>(a, vec, s); break;
      case EPI_SWIGLU: gemm_bf16<EPI_SWIGLU>(a, vec, s); break;
      case EPI_STORE: gemm_bf16<EPI_STORE>(a, vec, s); break;
    }
  } else {
    switch (epi) {
      case EPI_ACC: gemm_go<float, 64, 64, EPI_ACC>(a, vec, s); break;
      case EPI_RESID: gemm_go<float, 64, 64, EPI_RESID>(a, vec, s); break;
      case EPI_QKV:
        if (a.rope_l2 > 0.0)
          gemm_go<float, 64, 64, EPI_QKV_ROPE>(a, vec, s);
        else
          gemm_go<float, 64, 64, EPI_QKV>(a, vec, s);
        break;
      case EPI_QKV_ROPE: gemm_go<float, 64, 64, EPI_QKV_ROPE>(a, vec, s); break;
      case EPI_SWIGLU: gemm_go<float, 64, 64, EPI_SWIGLU>(a, vec, s); break;
      case EPI_STORE: gemm_go<float, 64, 64, EPI_STORE>(a, vec, s); break;
    }
  }
  return hipGetLastError();
}

template <typename T, int HD>
static void attn_go(const AttnArgs& a, const AttnPlan& p, int part, hipStream_t s) {
  if (part == 0) {
    if (sizeof(T) == 2 && HD == 128 && p.bq == kBQW)
      attn_pipe_kernel<8><<<p.nitems * a.Hd * batch_of(a), 512, 0, s>>>(a);
    else if (sizeof(T) == 2 && HD == 128)
      attn_pipe_kernel<4><<<p.nitems * a.Hd * batch_of(a), 256, 0, s>>>(a);
    else
      attn_kernel<T, HD><<<p.nitems * a.Hd * batch_of(a), 256, 0, s>>>(a);
  } else if (p.split) {
    const int64_t n = (int64_t)a.Hd * batch_of(a) * a.T * (HD / 4);
    attn_combine_kernel<T, HD><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  }
}

hipError_t launch_attention(Dtype dt, int hd, const AttnArgs& a, const AttnPlan& p, int part,
                            hipStream_t s) {
  if (a.T <= 0 || p.nitems <= 0) return hipSuccess;
  if (dt == BF16) {
    switch (hd) {
      case 16: attn_go<bf16, 16>(a, p, part, s); break;
      case 32: attn_go<bf16, 32>(a, p, part, s); break;
      case 64: attn_go<bf16, 64>(a, p, part, s); break;
      case 128: attn_go<bf16, 128>(a, p, part, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (hd) {
      case 16: attn_go<float, 16>(a, p, part, s); break;
      case 32: attn_go<float, 32>(a, p, part, s); break;
      case 64: attn_go<float, 64>(a, p, part, s); break;
      case 128: attn_go<float, 128>(a, p, part, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_fill32(void* p, uint32_t pattern, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  fill32_kernel<<<grid, 256, 0, s>>>((uint32_t*)p, pattern, n);
  return hipGetLastError();
}

// The 16-byte bf16 transpose when its alignment conditions hold and the grid
// fits; false: use the element-wise kernels.
static bool transpose16(Dtype dt, const void* in, void* out, int64_t R, int64_t Rw, int64_t C, int64_t ldi,
                        int64_t ldo, int64_t Z, int64_t zdiv, int64_t s1, int64_t s0, int64_t zs, hipStream_t s) {
  if (dt != BF16 || !aligned16(in) || !aligned16(out) || ((ldi | ldo | s1 | s0 | zs) & 7) != 0) return false;
  const int64_t gx = (Rw + 63) / 64, gy = (C + 63) / 64;
  if (gx > 0x7fffffff || gy > 65535 || Z > 65535) return false;
  transpose16_kernel<<<dim3((unsigned)gx, (unsigned)gy, (unsigned)Z), 256, 0, s>>>(
      (const bf16*)in, (bf16*)out, R, Rw, C, ldi, ldo, zdiv, s1, s0, zs);
  return true;
}

hipError_t launch_transpose(Dtype dt, const void* in, void* out, int64_t R, int64_t C, int64_t ldi,
                            int64_t ldo, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (transpose16(dt, in, out, R, R, C, ldi, ldo, 1, 1, 0, 0, 0, s)) return hipGetLastError();
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  if (dt == BF16)
    transpose_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)in, (bf16*)out, R, C, ldi, ldo);
  else
    transpose_kernel<float><<<grid, 256, 0, s>>>((const float*)in, (float*)out, R, C, ldi, ldo);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(Dtype dt, const void* in, void* out, int64_t R, int64_t Rp, int64_t C,
                                int64_t ldi, int64_t ldo, int64_t Z, int64_t zdiv, int64_t s1, int64_t s0,
                                hipStream_t s) {
  if (Rp <= 0 || C <= 0 || Z <= 0) return hipSuccess;
  if (Rp % 64 != 0 || Rp < R || zdiv <= 0 || Z > 65535 || (C + 63) / 64 > 65535) return hipErrorInvalidValue;
  if (transpose16(dt, in, out, R, Rp, C, ldi, ldo, Z, zdiv, s1, s0, Rp, s)) return hipGetLastError();
  const dim3 grid((unsigned)(Rp / 64), (unsigned)((C + 63) / 64), (unsigned)Z);
  if (dt == BF16)
    transpose_pad_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)in, (bf16*)out, R, Rp, C, ldi, ldo, zdiv, s1, s0);
  else
    transpose_pad_kernel<float><<<grid, 256, 0, s>>>((const float*)in, (float*)out, R, Rp, C, ldi, ldo, zdiv, s1,
                                                     s0);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(Dtype dt, const float* ab, const float* dg, void* dab, void* g, int64_t rows,
                             int64_t F, hipStream_t s) {
  const int64_t n = rows * F;
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
  if (dt == BF16)
    swiglu_bwd_kernel<bf16><<<grid, 256, 0, s>>>(ab, dg, (bf16*)dab, (bf16*)g, rows, F);
  else
    swiglu_bwd_kernel<float><<<grid, 256, 0, s>>>(ab, dg, (float*)dab, (float*)g, rows, F);
  return hipGetLastError();
}

int64_t gain_partial_floats(int64_t rows, int h) { return (rows + kGainRows - 1) / kGainRows * (int64_t)h; }

hipError_t launch_rmsnorm_bwd(Dtype dt, const void* x, const void* g, const float* dn, const void* res,
                              void* dx, float* rs, float* dgain, float* partial, int64_t rows, int h, float eps,
                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t nb = (rows + kGainRows - 1) / kGainRows;
  if (nb > 65535) return hipErrorInvalidValue;
  const dim3 rg((unsigned)((rows + 3) / 4)), cg((unsigned)((h + 255) / 256), (unsigned)nb);
  if (dt == BF16) {
    rmsnorm_bwd_kernel<bf16><<<rg, 256, 0, s>>>((const bf16*)x, (const bf16*)g, dn, (const bf16*)res,
                                               (bf16*)dx, rs, rows, h, eps);
    gain_grad_kernel<bf16><<<cg, 256, 0, s>>>((const bf16*)x, dn, rs, partial, rows, h);
  } else {
    rmsnorm_bwd_kernel<float><<<rg, 256, 0, s>>>((const float*)x, (const float*)g, dn, (const float*)res,
                                                (float*)dx, rs, rows, h, eps);
    gain_grad_kernel<float><<<cg, 256, 0, s>>>((const float*)x, dn, rs, partial, rows, h);
  }
  gain_sum_kernel<<<dim3((unsigned)((h + 255) / 256)), 256, 0, s>>>(partial, dgain, nb, h);
  return hipGetLastError();
}

hipError_t launch_spin(uint64_t ticks, hipStream_t s) {
  spin_kernel<<<1, 64, 0, s>>>(ticks);
  return hipGetLastError();
}

hipError_t launch_rope_inverse(float* v, int64_t rows, int heads, int hd, int64_t S, int64_t T, int64_t chunk,
                               int rank, int fold, double l2c, hipStream_t s) {
  const int64_t n = (int64_t)heads * rows * (hd / 4);
  if (n <= 0) return hipSuccess;
  rope_inverse_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(v, rows, heads, hd, S, T, chunk, rank, fold,
                                                                   l2c);
  return hipGetLastError();
}

hipError_t launch_kv_grad_reduce(const KvGradReduceArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.fold * 2 * a.hkd * a.batch * a.T * (a.hd / 4);
  if (n <= 0) return hipSuccess;
  kv_grad_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_qkv_grad_pack(Dtype dt, const float* dq, const float* dk, const float* dv, void* out,
                                int64_t rows, int hs, int ks, int hd, hipStream_t s) {
  const int64_t n = rows * ((hs + 2 * ks) / 4);
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (dt == BF16)
    qkv_grad_pack_kernel<bf16><<<grid, 256, 0, s>>>(dq, dk, dv, (bf16*)out, rows, hs, ks, hd);
  else
    qkv_grad_pack_kernel<float><<<grid, 256, 0, s>>>(dq, dk, dv, (float*)out, rows, hs, ks, hd);
  return hipGetLastError();
}

hipError_t launch_clock_probe(uint64_t* out, int n, uint64_t interval, hipStream_t s) {
  clock_probe_kernel<<<1, 64, 0, s>>>(out, n, interval);
  return hipGetLastError();
}

template <int HD>
hipError_t attn_bwd_hd(const AttnBwdArgs& a, int part, hipStream_t s) {
  if (part == 0) {
    const int64_t items = (int64_t)a.Hd * a.batch * a.T;
    attn_bwd_delta_kernel<HD><<<dim3((unsigned)((items + 3) / 4)), 256, 0, s>>>(a);
  } else if (part == 1) {
    attn_bwd_dkdv_kernel<HD><<<dim3((unsigned)((a.S + kBK2 - 1) / kBK2), a.Hkd, a.batch), 256, 0, s>>>(a);
  } else {
    attn_bwd_dq_kernel<HD><<<dim3((unsigned)a.dq_items, a.Hd, a.batch), 512, 0, s>>>(a);
    attn_bwd_dq_merge_kernel<HD><<<dim3((unsigned)((a.T + kBQ2 - 1) / kBQ2), a.Hd * a.batch), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(int hd, const AttnBwdArgs& a, int part, hipStream_t s) {
  if (hd == 128) return attn_bwd_hd<128>(a, part, s);
  if (hd == 64) return attn_bwd_hd<64>(a, part, s);
  return hipErrorInvalidValue;
}

}  // namespace tsp
