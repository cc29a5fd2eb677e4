// kernels.hip -- gfx950 (MI355X, CDNA4) kernels of the verify forward.
//
// One forward over S rows per sequence (the span [last, d1..dK], pegainfer
// page "DFlash speculative decoding", transaction section) runs:
//   embed -> per layer { QKV GEMM (+RMSNorm prologue, RoPE + KV-write
//   epilogue), attention, O GEMM (+residual), gate/up GEMM (+RMSNorm
//   prologue, SwiGLU epilogue), down GEMM (+residual) } -> LM-head GEMM with a
//   fused per-row argmax and, in its last workgroup, accept_greedy and the
//   cache advance.
//
// Numerics: bf16 weights are held as fp16 copies (exact for every value of
// magnitude 2^-17 .. 65504, which covers the weights); int4 weights are exact
// integers; the activations enter every GEMM once as fp16 (11 significant
// bits, above bf16's 8) and the MFMAs are fp16 x fp16 -> fp32; fp32
// accumulation, residual and softmax; fp16 KV cache, fp16 query and
// probabilities in attention.
// Row invariance: every row runs the same 16-row MFMA tiles, the same
// K-split per (N, K) and the same fixed-order reductions whatever S is, so a
// row's result does not depend on the other rows of the forward.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "internal.h"

namespace specv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Cross-workgroup hand-off inside one kernel.  Partial results are written
// and read with device-coherent (agent-scope) relaxed accesses, which bypass
// the per-XCD L2s' non-coherent copies, and a producer waits for its stores
// to complete before it signals the arrival counter.  This avoids the L2
// writeback + invalidate a full device-scope fence would issue in every
// workgroup.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {  // 8-byte aligned pair
  const unsigned long long v = __hip_atomic_load((const unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void st_dev2(float* p, float a, float b) {  // 8-byte aligned pair
  const unsigned long long v = (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Order-preserving key of (value, column): larger value wins, then the lower
// column.  Zero is below every key, so a zeroed slot is the neutral element.
__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal, as in the plain definition
  uint32_t u = __float_as_uint(v);
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

// ---------------------------------------------------------------- packing

// bf16 weights are packed as fp16: every bf16 value of magnitude 2^-17 ..
// 65504 is an fp16 value exactly (8 significant bits inside fp16's 11), the
// few smaller ones round with an absolute error <= 2^-25; a larger one (no
// fp16 value) sets *overflow, and the load is refused.
__global__ void k_pack_bf16(const uint16_t* __restrict__ src, int rows, int cols, u32x4* __restrict__ dst,
                            int kind, int row0, int hd, uint32_t* __restrict__ overflow) {
  const int chunks = cols / 8;
  const size_t total = (size_t)rows * chunks;
  bool over = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int s = (int)(i / chunks), kc = (int)(i % chunks);
    int n;
    if (kind == 0) n = row0 + s;
    else if (kind == 1) n = row0 + rope_pair_row(s, hd);
    else n = row0 + 2 * s;
    const uint16_t* v = src + (size_t)s * cols + (size_t)kc * 8;
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf16_bits_to_f32(v[e]);
      h[e] = (_Float16)f;
      over |= __builtin_isinf((float)h[e]) && !__builtin_isinf(f);
    }
    const int tile = n >> 4, r = n & 15, step = kc >> 2, g = kc & 3;
    dst[((size_t)tile * (cols / 32) + step) * 64 + g * 16 + r] = __builtin_bit_cast(u32x4, h);
  }
  if (over) atomicOr(overflow, 1u);
}

// One thread per (source row, 128-input group): 64 source bytes become one
// dword per (step d, lane group gq) of the fragment, plus the group's scale.
__global__ void k_pack_int4(const uint8_t* __restrict__ q4, const uint16_t* __restrict__ sc, int rows, int cols,
                            uint32_t* __restrict__ dst, uint16_t* __restrict__ dsc, int kind, int row0, int hd) {
  const int KG = cols / 128;
  const size_t total = (size_t)rows * KG;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int s = (int)(i / KG), g = (int)(i % KG);
    int n;
    if (kind == 0) n = row0 + s;
    else if (kind == 1) n = row0 + rope_pair_row(s, hd);
    else n = row0 + 2 * s;
    const int tile = n >> 4, r = n & 15;
    const uint32_t* src = (const uint32_t*)(q4 + (size_t)s * (cols / 2) + (size_t)g * 64);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const uint32_t w = src[d * 4 + gq];  // nibble e (input 32d + 8gq + e) at bits 4e
        uint32_t out = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = ((w >> (4 * e)) & 0xFu) ^ 0x8u;  // two's complement -> offset q + 8
          out |= u << ((e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1));
        }
        dst[(((size_t)tile * KG + g) * 64 + gq * 16 + r) * 4 + d] = out;
      }
    dsc[((size_t)tile * 16 + r) * KG + g] = sc[(size_t)s * KG + g];
  }
}

__global__ void k_fill_u32(uint32_t* __restrict__ dst, uint32_t value, size_t count) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = value;
}

// -------------------------------------------------------------- embedding

// One workgroup per row: x = E[token] in fp32, plus the sum of squares of
// every 16-column group (the format the RMSNorm prologues consume).
__global__ __launch_bounds__(256) void k_embed(EmbedParams P) {
  const int r = blockIdx.x;
  {
    const int b = r / P.S, seq = P.seq_ids[b];
    const int len = P.kv_len[seq], pos = len + (r - b * P.S);
    const int32_t* row = P.bt + (size_t)seq * P.bt_stride;
    if (threadIdx.x == 0) {
      P.rowinfo[2 * r] = pos;
      P.rowinfo[2 * r + 1] = row[pos >> 4];
    }
    if (r == b * P.S) {  // the sequence's first row copies its blocks, by slot, for attention
      const int nb = (len + P.S + 15) >> 4;
      for (int i = threadIdx.x; i < nb; i += blockDim.x) P.slotbt[(size_t)b * P.bt_stride + i] = row[i];
    }
  }
  const int tok = P.tokens[r];
  const int H = P.H, ng = H / 16;
  const uint16_t* e = P.emb + (size_t)tok * H;
  for (int c0 = 0; c0 < H; c0 += 256) {
    const int c = c0 + threadIdx.x;
    if (c0 + (int)(threadIdx.x & ~63) < H) {  // whole waves in or out
      const float v = bf16_bits_to_f32(e[c]);
      P.x[(size_t)r * H + c] = v;
      float t = v * v;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) t += __shfl_xor(t, o);
      if ((threadIdx.x & 15) == 0) P.ss[(size_t)r * ng + c / 16] = t;
    }
  }
}

// ------------------------------------------------------------ skinny GEMM
//
// Y[R, N] = A'[R, K] W^T with A' = RMSNorm(A) (optional) rounded to fp16.  A
// workgroup (4 waves) owns 64 output columns x one K slice of NK*32 inputs;
// wave w owns the 16-column tile 4*nb + w.  Each wave first issues all NK
// fragment loads of its weights (contiguous NK KiB, streamed with
// non-temporal loads), then stages A for 16 rows of the slice into LDS in the
// MFMA A-operand order, then runs NK MFMA 16x16x32 f16.  The split
// partial sums go to memory; the last workgroup of a column block to arrive
// (counted with an atomic) adds the slices in slice order and runs the
// epilogue, so the result is deterministic and independent of R.
// Workgroup ids are mapped so every slice of a column block sits on the same
// XCD (ids are dealt round-robin over the 8 XCDs), keeping the partial sums
// in one L2.

// SB slices per gather round and U pairs per thread (eight and two keep the
// split-K kernel's registers, and so its occupancy, low).
template <int EPI, int CT, int SB = 8, int U = 2>
__device__ void gemm_epilogue(const GemmParams& P, int nb, float* sbuf);

// 16-column tiles per wave: int4 fragments are a quarter the bytes of bf16
// ones, so an int4 wave takes four tiles (a 256-column block per workgroup)
// to stream as many weight bytes per staged activation tile.
constexpr int gemm_tiles_per_wave(int fmt) { return fmt == FMT_INT4 ? 4 : 1; }

// RMSNorm statistics: the producer of a residual row writes the sum of
// squares of every 16-column group; a consumer sums them with 16 lanes per
// row, lane j taking groups j, j + 16, ... in increasing order, then a fixed
// xor tree -- the same order for every kernel and any number of rows.
constexpr int kSsChunk = 8;  // partial-sum loads in flight per lane
__device__ __forceinline__ float rstd_finish(float acc, float inv_dim, float eps) {
#pragma clang fp contract(off)
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  return 1.0f / sqrtf(acc * inv_dim + eps);
}
__device__ __forceinline__ float rstd16(const float* ss, int ss_n, int r, int R, int j, float inv_dim, float eps) {
#pragma clang fp contract(off)
  float acc = 0.0f;
  for (int i0 = 0; i0 * 16 < ss_n; i0 += kSsChunk) {
    float v[kSsChunk];
#pragma unroll
    for (int i = 0; i < kSsChunk; ++i) {
      const int q = j + 16 * (i0 + i);
      v[i] = (r < R && q < ss_n) ? ss[(size_t)r * ss_n + q] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kSsChunk; ++i) acc += v[i];
  }
  return rstd_finish(acc, inv_dim, eps);
}

// Offset nibbles -> exact fp16 q: (1024 + u) - 1032 in packed fp16.
// Eight int4 weights of a fragment dword as fp16 q = u - 8 (u the stored
// nibble; the low halves hold nibbles 0-3, the high halves 4-7).  SHIFTLESS:
// the sequence of dequant8_ao below with the AND-OR left to the compiler
// (two instructions with literal operands, no register for the constants);
// otherwise one shift, AND-OR and add per nibble pair, for the split-K QKV
// kernel, which the other sequence takes past 256 registers.  Both give the
// same values.
template <bool SHIFTLESS>
__device__ __forceinline__ f16x8 dequant8(uint32_t x) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  if constexpr (SHIFTLESS) {
    const uint32_t x8 = x >> 8;
    const uint32_t m0 = (x & 0x000F000Fu) | 0x64006400u, m1 = (x & 0x00F000F0u) | 0x64006400u;
    const uint32_t m2 = (x8 & 0x000F000Fu) | 0x64006400u, m3 = (x8 & 0x00F000F0u) | 0x64006400u;
    const h2 sc = {(_Float16)0.0625f, (_Float16)0.0625f}, off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const h2 v0 = __builtin_bit_cast(h2, m0) - off, v2 = __builtin_bit_cast(h2, m2) - off;
    const h2 v1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, m1), sc, off16);
    const h2 v3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, m3), sc, off16);
    return (f16x8){v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
  } else {
    f16x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
      const h2 v = __builtin_bit_cast(h2, o) - off;
      r[2 * j] = v[0];
      r[2 * j + 1] = v[1];
    }
    return r;
  }
}

// (x & mask) | 0x64006400 in one VOP3 instruction (which takes no literal:
// the mask comes in a scalar register, the fp16 exponent pattern in a vector
// register).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(0x64006400u));
  return r;
}

__device__ __forceinline__ f16x8 dequant8_ao(uint32_t x) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  // The eight values of dequant8 in fewer instructions.  A nibble u = q + 8
  // placed in bits 0-3 of an fp16 with exponent field 25 (0x6400) is the
  // exact value 1024 + u; placed in bits 4-7 it is 1024 + 16 u, and
  // (1024 + 16 u) / 16 - 72 = u - 8 with no rounding.  So the nibble pairs
  // (j, j + 4) of x at bits 4j, 16 + 4j take one AND-OR each, with one shift
  // by 8 for j = 2, 3, and one packed add or fma per pair.  The exponent
  // pattern takes a vector register, which the split-K kernel, at the
  // register limit of two waves per SIMD, cannot spare: it takes dequant8.
  const uint32_t x8 = x >> 8;
  const uint32_t m0 = and_or(x, 0x000F000Fu), m1 = and_or(x, 0x00F000F0u);
  const uint32_t m2 = and_or(x8, 0x000F000Fu), m3 = and_or(x8, 0x00F000F0u);
  const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 sc = {(_Float16)0.0625f, (_Float16)0.0625f}, off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const h2 v0 = __builtin_bit_cast(h2, m0) - off, v2 = __builtin_bit_cast(h2, m2) - off;
  const h2 v1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, m1), sc, off16);
  const h2 v3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, m3), sc, off16);
  return (f16x8){v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

template <int NK, int EPI, int FMT>
__global__ __launch_bounds__(256) void k_gemm(GemmParams P) {
  static_assert(FMT == FMT_BF16 || NK % 4 == 0, "int4 slices hold whole 128-input groups");
  constexpr int NF = FMT == FMT_INT4 ? NK / 4 : NK;  // weight fragments per tile per slice
  constexpr int CT = gemm_tiles_per_wave(FMT);       // 16-column tiles per wave
  constexpr int UNITS = 16 * NK * 4;          // (row, step, lane group) units of 8 inputs per 16-row chunk
  constexpr int UPT = (UNITS + 255) / 256;    // units per thread
  const int NB = (P.N + 64 * CT - 1) / (64 * CT), ns = P.nslices;
  const int id = blockIdx.x, xcd = id & 7, loc = id >> 3;
  const int nb = (loc / ns) * 8 + xcd, sl = loc % ns;
  if (nb >= NB) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int k0 = sl * NK * 32;
  const int tile0 = (nb * 4 + wave) * CT;  // this wave's first tile; tiles past N (a ragged last block) idle

  __shared__ u32x4 sA[NK * 2 * 64];
  __shared__ float sR[kMaxRows];
  __shared__ float sG[NK * 32];
  __shared__ int sLast;

  // Loads are issued in the order they are needed: the RMSNorm partial sums
  // and gain, then A of the first 16 rows, and the weights last, so the
  // prologue's arithmetic overlaps the weights' DRAM latency.
  const int ss_row = tid >> 4, ss_part = tid & 15;
  if (P.ss)
    for (int e = tid; e < NK * 32; e += 256) sG[e] = P.gain[k0 + e];
  f32x4 pa[UPT][2];
  auto load_a = [&](int m0) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * 256;
      const int g = u & 3, j = (u >> 2) % NK, row = u / (4 * NK);
      const int r = m0 + row;
      if (u < UNITS && r < P.R) {
        const f32x4* src = (const f32x4*)(P.A + (size_t)r * P.lda + k0 + j * 32 + g * 8);
        pa[i][0] = src[0];
        pa[i][1] = src[1];
      } else {
        pa[i][0] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        pa[i][1] = pa[i][0];
      }
    }
  };
  load_a(0);

  // bf16: one fragment per 32-input step; int4: one per 128-input group.
  u32x4 b[CT][NF];
  float gs[CT][FMT == FMT_INT4 ? NF : 1];  // int4: this lane's column's group scales
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int tile = tile0 + c;
    if (tile * 16 < P.N) {
      const u32x4* wp = (const u32x4*)P.W + ((size_t)tile * (P.K / (32 * NK / NF)) + (size_t)sl * NF) * 64 + lane;
#pragma unroll
      for (int j = 0; j < NF; ++j) b[c][j] = __builtin_nontemporal_load(wp + j * 64);
      if constexpr (FMT == FMT_INT4) {
        const uint16_t* sp = P.scales + ((size_t)tile * 16 + (lane & 15)) * (P.K / 128) + (size_t)sl * NF;
#pragma unroll
        for (int g = 0; g < NF; ++g) gs[c][g] = bf16_bits_to_f32(sp[g]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NF; ++j) b[c][j] = (u32x4){0u, 0u, 0u, 0u};
      if constexpr (FMT == FMT_INT4) {
#pragma unroll
        for (int g = 0; g < NF; ++g) gs[c][g] = 0.0f;
      }
    }
  }

  if (P.ss) {
    // rstd of every row, 16 lanes per row (rstd16)
    for (int pass = 0; pass * 16 < P.R; ++pass) {
      const int r = pass * 16 + ss_row;
      const float rs = rstd16(P.ss, P.ss_n, r, P.R, ss_part, P.inv_dim, P.eps);
      if (ss_part == 0) sR[r] = r < P.R ? rs : 0.0f;
    }
    __syncthreads();
  }

  for (int m0 = 0; m0 < P.R; m0 += 16) {
    // A' for 16 rows x NK*32 inputs into LDS in the MFMA A-operand order, as fp16.
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * 256;
      if (u >= UNITS) continue;
      const int g = u & 3, j = (u >> 2) % NK, row = u / (4 * NK);
      float v[8] = {pa[i][0].x, pa[i][0].y, pa[i][0].z, pa[i][0].w, pa[i][1].x, pa[i][1].y, pa[i][1].z, pa[i][1].w};
      if (P.ss) {
        const int r = m0 + row;
        const float rs = r < P.R ? sR[r] : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (v[e] * rs) * sG[j * 32 + g * 8 + e];
      }
      f16x8 hi;  // fp16: the operand type of the fp16 MFMA on the exact fp16 weights (int4: exact q)
#pragma unroll
      for (int e = 0; e < 8; ++e) hi[e] = (_Float16)v[e];
      sA[(j * 2) * 64 + g * 16 + row] = __builtin_bit_cast(u32x4, hi);
    }
    __syncthreads();
    if (m0 + 16 < P.R) load_a(m0 + 16);  // the next chunk's A loads fly during this chunk's MFMA
    f32x4 acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (FMT == FMT_INT4) {
      // Per group: exact integer weights times the activation pair, summed
      // over the group's four steps in fp32, then scaled by the column's
      // group scale and added in group order.  The A fragments of a step
      // serve every tile of the wave.
#pragma unroll
      for (int gi = 0; gi < NF; ++gi) {
        f32x4 t[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) t[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int j = gi * 4 + d;
          const f16x8 ah = __builtin_bit_cast(f16x8, sA[(j * 2) * 64 + lane]);
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            // Opaque per row chunk, so the dequantised operands are rebuilt
            // from the packed nibbles each time instead of being hoisted out
            // of the chunk loop into 4x the registers.
            uint32_t w = b[c][gi][d];
            asm volatile("" : "+v"(w));
            const f16x8 bq = dequant8<EPI != EPI_QKV>(w);
            t[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, t[c], 0, 0, 0);
          }
        }
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[c][i] = __builtin_fmaf(t[c][i], gs[c][gi], acc[c][i]);  // one rounding
      }
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const f16x8 ah = __builtin_bit_cast(f16x8, sA[(j * 2) * 64 + lane]);
#pragma unroll
        for (int c = 0; c < CT; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(f16x8, b[c][j]), acc[c], 0, 0, 0);
      }
    }
    // D layout: lane holds column lane%16 of rows 4*(lane/16) + i.
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int col = (tile0 + c) * 16 + (lane & 15);
      if (col < P.N)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m0 + (lane >> 4) * 4 + i;
          if (r < P.R) st_dev(P.part + ((size_t)sl * P.R + r) * P.N + col, acc[c][i]);
        }
    }
    __syncthreads();  // sA is restaged for the next 16 rows
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) {
    const unsigned old = atomicAdd(&P.cnt[nb], 1u);
    sLast = (old == (unsigned)(ns - 1));
  }
  __syncthreads();
  if (!sLast) return;
  if (tid == 0) P.cnt[nb] = 0u;  // ready for the next launch
  // int4 down runs 50 slices: 16 per gather round (four rounds, not seven)
  gemm_epilogue<EPI, CT, FMT == FMT_INT4 ? 16 : 8>(P, nb, (float*)sA);
}

// The epilogue's column pairs of block nb (64*CT columns): pair idx = (row
// idx/(32CT), columns nb*64CT + 2*(idx%(32CT)) + {0,1}), summed over the K
// slices in slice order; pairs past N (a ragged last block) are skipped, 64
// columns at a time.  Each thread takes U pairs at a time and issues every
// slice load of them (up to SB slices per round) before the first add, so the
// gather costs one memory round trip per U pairs and per SB slices.  Every
// 32 consecutive pairs are 64 columns of one row (the shuffle groups of the
// epilogues).
template <int CT, int SB = 8, int U = 2, class F>
__device__ __forceinline__ void for_pairs(const GemmParams& P, int nb, F&& f) {
#pragma clang fp contract(off)
  constexpr int PR = 32 * CT;
  const int n = P.R * PR, ns = P.nslices;
  const unsigned stride = (unsigned)P.R * (unsigned)P.N;  // floats; the partial buffer is < 4 GiB
  for (int base = 0; base < n; base += U * 256) {
    float v0[U], v1[U];
    unsigned off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * 256 + threadIdx.x;
      const int c = nb * 64 * CT + 2 * (idx % PR);
      v0[u] = v1[u] = 0.0f;
      ok[u] = idx < n && c < P.N;
      off[u] = (unsigned)(idx / PR) * (unsigned)P.N + (unsigned)c;
    }
    for (int s0 = 0; s0 < ns; s0 += SB) {
      float2 t[U][SB];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (ok[u] && s0 + i < ns) t[u][i] = ld_dev2(P.part + (off[u] + (unsigned)(s0 + i) * stride));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (ok[u] && s0 + i < ns) {
            v0[u] += t[u][i].x;
            v1[u] += t[u][i].y;
          }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * 256 + threadIdx.x;
      if (ok[u]) f(idx, idx / PR, nb * 64 * CT + 2 * (idx % PR), v0[u], v1[u]);
    }
  }
}

// Per column-pair epilogue arithmetic, shared by the split-K and the
// one-pass GEMMs so that both give bit-identical results (contraction off:
// every product and sum rounds on its own, whatever the surrounding code).

// The (cos, sin) pair RoPE applies to output column c of a row at position
// pos (a q or k column), or (0, 0) for a v column or a recurrent layer.
__device__ __forceinline__ float2 rope_cs(const GemmParams& P, int c, int pos) {
  const int hd = P.hd, DQ = P.n_q * hd, DK = P.n_kv * hd;
  if (P.rec_kv || c >= DQ + DK) return make_float2(0.0f, 0.0f);
  const int local = c < DQ ? c : c - DQ, j = (local % hd) >> 1;
  return *(const float2*)(P.rope + ((size_t)pos * (hd / 2) + j) * 2);
}

// RoPE on the pair (d, d + hd/2) stored interleaved, then q (fp32) or the
// K / V cache rows (fp16) at the row's position.
// pos: the row's absolute position; blk: the KV block holding it; cs2: the
// column's rope_cs.
__device__ __forceinline__ void qkv_pair_cs(const GemmParams& P, int r, int c, float v0, float v1, int pos,
                                            int blk, float2 cs2) {
#pragma clang fp contract(off)
  const int hd = P.hd, half = hd / 2;
  const int DQ = P.n_q * hd, DK = P.n_kv * hd;
  const int slot = pos & 15;
  if (P.rec_kv) {
    // a recurrent layer: queries, keys and values unrotated, no cache row
    if (c < DQ + DK) {
      const int local = c < DQ ? c : c - DQ;
      const int head = local / hd, j = (local % hd) >> 1;
      float* dst = c < DQ ? P.q + (size_t)r * DQ : P.rec_kv + (size_t)r * 2 * DK;
      dst[head * hd + j] = v0;
      dst[head * hd + j + half] = v1;
    } else {
      float* dst = P.rec_kv + (size_t)r * 2 * DK + DK + (c - DQ - DK);
      dst[0] = v0;
      dst[1] = v1;
    }
    return;
  }
  // a sliding-window layer keeps its KV rows in the sequence's ring
  if (P.ring_nb && c >= DQ) blk = P.seq_ids[r / P.S] * P.ring_nb + ((pos % P.ring_w) >> 4);
  if (c < DQ + DK) {
    const int local = c < DQ ? c : c - DQ;
    const int head = local / hd, j = (local % hd) >> 1;
    const float cs = cs2.x, sn = cs2.y;
    const float o0 = v0 * cs - v1 * sn, o1 = v0 * sn + v1 * cs;
    if (c < DQ) {
      if (P.q16) {
        _Float16* qr = P.q16 + (size_t)r * DQ + head * hd;
        qr[j] = (_Float16)o0;
        qr[j + half] = (_Float16)o1;
      } else {
        float* qr = P.q + (size_t)r * DQ + head * hd;
        qr[j] = o0;
        qr[j + half] = o1;
      }
    } else {
      _Float16* kr = P.kpool + (((size_t)blk * P.n_kv + head) * 16 + slot) * hd;
      kr[j] = (_Float16)o0;
      kr[j + half] = (_Float16)o1;
    }
  } else {
    const int local = c - DQ - DK;
    const int head = local / hd, d = local % hd;
    _Float16* vb = P.vpool + ((size_t)blk * P.n_kv + head) * hd * 16;
    vb[(size_t)d * 16 + slot] = (_Float16)v0;
    vb[(size_t)(d + 1) * 16 + slot] = (_Float16)v1;
  }
}

__device__ __forceinline__ void qkv_pair_at(const GemmParams& P, int r, int c, float v0, float v1, int pos,
                                            int blk) {
  qkv_pair_cs(P, r, c, v0, v1, pos, blk, rope_cs(P, c, pos));
}
__device__ __forceinline__ void qkv_pair(const GemmParams& P, int r, int c, float v0, float v1) {
  qkv_pair_at(P, r, c, v0, v1, P.rowinfo[2 * r], P.rowinfo[2 * r + 1]);
}

// x += (v0, v1) given x's current pair; returns the pair's sum of squares
// of the new residual.
__device__ __forceinline__ float resid_pair_x(const GemmParams& P, int r, int c, float v0, float v1, float2 x) {
#pragma clang fp contract(off)
  x.x = x.x + v0;
  x.y = x.y + v1;
  *(float2*)(P.x + (size_t)r * P.N + c) = x;
  return x.x * x.x + x.y * x.y;
}
__device__ __forceinline__ float resid_pair(const GemmParams& P, int r, int c, float v0, float v1) {
  return resid_pair_x(P, r, c, v0, v1, *(const float2*)(P.x + (size_t)r * P.N + c));
}

// Sum over the 8 pairs (16 columns) held by an aligned group of 8 lanes;
// every lane of the group must be active.
__device__ __forceinline__ float sum8(float t) {
#pragma clang fp contract(off)
  t += __shfl_xor(t, 4);
  t += __shfl_xor(t, 2);
  t += __shfl_xor(t, 1);
  return t;
}

// Prepared A (k_prep's layout, fp16, nch = ceil(R/16) chunks) written by a
// producer: element (row r, input k) sits at fp16 index
// ((k/32 * nch + r/16) * 64 + r%16 + 16 * (k%32/8)) * 8 + k%8; the rounding
// is k_prep's, so the consumer sees the same operands.
__device__ __forceinline__ size_t prep_index(int nch, int r, int k) {
  return (((size_t)(k >> 5) * nch + (r >> 4)) * 64 + (r & 15) + 16 * ((k >> 3) & 3)) * 8 + (k & 7);
}
__device__ __forceinline__ void prep_store1(void* af, int nch, int r, int k, float v) {
  ((_Float16*)af)[prep_index(nch, r, k)] = (_Float16)v;
}
// k even: the pair (k, k + 1) is one 4-byte word
__device__ __forceinline__ void prep_store2(void* af, int nch, int r, int k, float v0, float v1) {
  const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
  *(uint32_t*)((_Float16*)af + prep_index(nch, r, k)) =
      (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
}

__device__ __forceinline__ float swiglu_val(float g, float u) {
#pragma clang fp contract(off)
  return (g / (1.0f + expf(-g))) * u;
}
__device__ __forceinline__ void swiglu_pair(const GemmParams& P, int r, int c, float g, float u) {
  const float v = swiglu_val(g, u);
  const size_t i = (size_t)r * (P.N >> 1) + (c >> 1);
  P.h[i] = v;
  if (P.h16) P.h16[i] = (_Float16)v;
}

template <int CT, int SB, int U>
__device__ void epi_qkv(const GemmParams& P, int nb) {
  for_pairs<CT, SB, U>(P, nb, [&](int, int r, int c, float v0, float v1) { qkv_pair(P, r, c, v0, v1); });
}

template <int CT, int SB, int U>
__device__ void epi_resid(const GemmParams& P, int nb) {
  const int NG = P.N >> 4;  // RMSNorm partial sums: one per 16 columns
  for_pairs<CT, SB, U>(P, nb, [&](int idx, int r, int c, float v0, float v1) {
    const float t = sum8(resid_pair(P, r, c, v0, v1));
    if ((idx & 7) == 0) P.ss_out[(size_t)r * NG + (c >> 4)] = t;
  });
}

// Above 16 rows the down GEMM (the many-row kernel) reads the prepared
// layout: h is also written there (af_out), only on that path.
__device__ __forceinline__ void swiglu_prep_pair(const GemmParams& P, int r, int c, float g, float u) {
  const float v = swiglu_val(g, u);
  P.h[(size_t)r * (P.N >> 1) + (c >> 1)] = v;
  if (P.af_out) prep_store1(P.af_out, (P.R + 15) >> 4, r, c >> 1, v);
}
template <int CT, int SB, int U>
__device__ void epi_swiglu(const GemmParams& P, int nb) {
  for_pairs<CT, SB, U>(P, nb, [&](int, int r, int c, float g, float u) { swiglu_prep_pair(P, r, c, g, u); });
}

// Sampled rows (step temperature > 0): a row draws its token from
// softmax(logit / T) as argmax_v (logit_v / T + g_v), g_v = -log(-log u_v)
// (the Gumbel-max rule), so the accept stage's argmax machinery serves both
// modes.  u_v comes from Philox4x32-10 (Salmon et al., SC 2011: ten rounds of
// two 32 x 32 -> 64-bit products, multipliers 0xD2511F53 and 0xCD9E8D57, key
// advanced by 0x9E3779B9 and 0xBB67AE85) with key = the seed and counter =
// (v / 4, the row's position, the sequence id, 0), word v % 4: a draw depends
// on (seed, sequence, position, v) alone, so a plain decode of the same
// prefix draws the same token.  u = (top 23 bits + 1/2) * 2^-23.
struct Sampling {
  float temp;
  uint32_t k0, k1;
};

__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                          uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return (u32x4){c0, c1, c2, c3};
}

__device__ __forceinline__ float gumbel_of(uint32_t x) {
#pragma clang fp contract(off)
  const float u = ((float)(x >> 9) + 0.5f) * (1.0f / 8388608.0f);
  return -logf(-logf(u));
}

// The keys of the pair (c, c + 1), c even, of row r: argmax keys of the
// logits (greedy) or of the sampled scores.  pos: the row's position.
__device__ __forceinline__ void lm_pair_keys(const GemmParams& P, const Sampling& sm, int r, int c, float v0,
                                             float v1, int pos, unsigned long long& k0, unsigned long long& k1) {
#pragma clang fp contract(off)
  if (P.logits) *(float2*)(P.logits + (size_t)r * P.N + c) = make_float2(v0, v1);
  if (v0 != v0 || v1 != v1) atomicOr(P.status, 1);
  if (sm.temp > 0.0f) {
    const int seq = P.seq_ids[r / P.S];
    const u32x4 w = philox10((uint32_t)c >> 2, (uint32_t)pos, (uint32_t)seq, 0u, sm.k0, sm.k1);
    const int j = c & 3;  // 0 or 2
    v0 = v0 / sm.temp + gumbel_of(j ? w[2] : w[0]);
    v1 = v1 / sm.temp + gumbel_of(j ? w[3] : w[1]);
  }
  k0 = argmax_key(v0, c);
  k1 = argmax_key(v1, c + 1);
}

__device__ __forceinline__ Sampling load_sampling(const GemmParams& P) {
  Sampling s;
  s.temp = P.step->temp;
  s.k0 = P.step->seed_lo;
  s.k1 = P.step->seed_hi;
  return s;
}

// After a workgroup's row maxima are in: the last of nblk workgroups reads
// them, runs accept_greedy per sequence and advances the cache lengths.
__device__ void lm_finish(const GemmParams& P, int nblk, float* sbuf) {
  __shared__ int sFinal;
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = atomicAdd(P.lm_cnt, 1u);
    sFinal = (old == (unsigned)(nblk - 1));
  }
  __syncthreads();
  if (!sFinal) return;
  int* arg = (int*)sbuf;
  __shared__ int sNan;
  for (int r = threadIdx.x; r < P.R; r += blockDim.x) {
    const unsigned long long k = atomicExch(&P.argkey[r], 0ull);
    arg[r] = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
  }
  // every workgroup's NaN flag is in (they arrived after their stores landed)
  if (threadIdx.x == 0) sNan = __hip_atomic_load(P.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1;
  __syncthreads();
  // A NaN row leaves every cache length where it was: the forward failed, and
  // the host keeps its mirror of the lengths unchanged too.
  const int mode = sNan ? (int)MODE_NO_COMMIT : *P.mode, S = P.S;
  for (int b = threadIdx.x; b < P.n_seq; b += blockDim.x) {
    const int row0 = b * S;
    int m;
    if (mode == MODE_COMMIT_ALL) {
      m = S - 1;
    } else {
      // accept_greedy over the sequence's own drafts; padding rows never count
      const int kb = min(S - 1, max(0, P.kd[b]));
      m = 0;
      while (m < kb && P.tokens[row0 + m + 1] == arg[row0 + m]) ++m;
    }
    const int seq = P.seq_ids[b];
    if (mode == MODE_COMMIT_ALL) P.kv_len_w[seq] += S;
    else if (mode == MODE_VERIFY) P.kv_len_w[seq] += m + 1;
    if (P.rec_slot && mode != MODE_NO_COMMIT) {
      // the recurrent layers wrote this forward's per-row states into the set
      // the committed state is not in; the state after the last kept row
      // becomes the committed one (no copy, no second forward)
      const int old = P.rec_slot[seq];
      const int set = old < 0 ? 0 : 1 - (old >> 4);
      P.rec_slot[seq] = set * 16 + (mode == MODE_COMMIT_ALL ? S - 1 : m);
    }
    int32_t* res = P.result + 1 + b * (S + 1);
    res[0] = m;
    for (int i = 0; i < S; ++i) res[1 + i] = arg[row0 + i];
  }
  if (threadIdx.x == 0) {
    P.result[0] = atomicExch(P.status, 0);
    *P.lm_cnt = 0u;
  }
}

template <int CT, int SB, int U>
__device__ void epi_lm(const GemmParams& P, int nb, float* sbuf) {
  const Sampling sm = load_sampling(P);
  for_pairs<CT, SB, U>(P, nb, [&](int idx, int r, int c, float v0, float v1) {
    unsigned long long k0, k1;
    lm_pair_keys(P, sm, r, c, v0, v1, P.rowinfo[2 * r], k0, k1);
    unsigned long long k = k0 > k1 ? k0 : k1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      const unsigned long long t = __shfl_xor(k, o);
      k = t > k ? t : k;
    }
    if ((idx & 31) == 0) atomicMax(&P.argkey[r], k);
  });
  lm_finish(P, (P.N + 64 * CT - 1) / (64 * CT), sbuf);
}

template <int EPI, int CT, int SB, int U>
__device__ void gemm_epilogue(const GemmParams& P, int nb, float* sbuf) {
  if constexpr (EPI == EPI_QKV) epi_qkv<CT, SB, U>(P, nb);
  else if constexpr (EPI == EPI_RESID) epi_resid<CT, SB, U>(P, nb);
  else if constexpr (EPI == EPI_SWIGLU) epi_swiglu<CT, SB, U>(P, nb);
  else epi_lm<CT, SB, U>(P, nb, sbuf);
}

// Slice sums of the many-row GEMM (above 16 rows) and its epilogue, as a
// kernel of its own: one (row, column pair) per thread, so the gather has the
// whole chip's loads in flight instead of one workgroup per column block
// walking 128 rows.  Pair (r, p) is row r, columns 2p and 2p + 1; a row's
// pairs are padded to a multiple of 8 so that every aligned group of 8 lanes
// (one RMSNorm partial sum, 16 columns) holds pairs of one row.  The slices
// are added in slice order from zero, as in the split-K kernel's gather.
template <int EPI>
__global__ __launch_bounds__(256) void k_gather(GemmParams P) {
#pragma clang fp contract(off)
  static_assert(EPI != EPI_LM, "the LM head keeps its in-kernel gather (row maxima, accept stage)");
  const int PW = ((P.N >> 1) + 7) & ~7;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int r = idx / PW, p = idx - r * PW, c = 2 * p;
  const bool ok = r < P.R && c < P.N;
  float v0 = 0.0f, v1 = 0.0f;
  if (ok) {
    const size_t stride = (size_t)P.R * P.N;
    const float* src = P.part + (size_t)r * P.N + c;
    for (int s0 = 0; s0 < P.nslices; s0 += 8) {
      float2 t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < P.nslices) t[i] = *(const float2*)(src + (size_t)(s0 + i) * stride);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < P.nslices) {
          v0 += t[i].x;
          v1 += t[i].y;
        }
    }
  }
  if constexpr (EPI == EPI_QKV) {
    if (ok) qkv_pair(P, r, c, v0, v1);
  } else if constexpr (EPI == EPI_RESID) {
    const float t = sum8(ok ? resid_pair(P, r, c, v0, v1) : 0.0f);  // every lane of the group shuffles
    if (ok && (p & 7) == 0) P.ss_out[(size_t)r * (P.N >> 4) + (c >> 4)] = t;
  } else {
    if (ok) swiglu_prep_pair(P, r, c, v0, v1);
  }
}

// ------------------------------------------------ many-row GEMM (17..128 rows)
//
// fp16 weights, prepared A (k_prep's layout, or a producer's).  The 32x32x16
// MFMA: on gfx950 it issues twice the flops per cycle of the 16x16x32 form
// the one-pass kernels use (measured: 2.4 against 1.3 PFLOP/s of fp16 on
// register operands), which matters at 128 rows (256 flop per weight
// element, against at most 32 on the one-pass paths).  A workgroup of four waves owns a block of 64*CT columns (TB = 4*CT
// packed 16-column tiles, NP = 2*CT MFMA column tiles of 32) and every row:
// wave w rows 32w..32w+31, its NP accumulators (32x32 each) in registers.
// It walks the K range of slice sl (ksl steps of 32 inputs).  A step's
// weights (TB packed fragments of 1 KB) are loaded by the 256 lanes, CT
// 16-byte words each, and pass through a two-slot LDS ring (one barrier per
// step: a slot is rewritten two steps later, after every wave has passed the
// barrier between); each wave reads its B operands from there and its two A
// operands (the step's two 16-input halves) straight from the prepared
// layout.  Both are issued PD steps ahead into register rings.
//
// Operand gathers: the 32x32x16 A operand of rows 32w.. and inputs
// 16h..16h+15 of a step gives lane l row l%32 and inputs 8*(l/32).., which
// in the prepared layout (16-row chunks, lane r + 16g: row r, inputs 8g..)
// is word (l%16) + 16*(2h + l/32) of chunk 2w + (l/16)%2; the B operand of
// columns 32p.. likewise is word (l%16) + 16*(2h + l/32) of packed tile
// 2p + (l/16)%2.  D: lane l value v is row 8*(v/4) + 4*(l/32) + v%4, column
// l%32.  One slice (ns = 1): the epilogue runs here, on the block's outputs
// staged in LDS; several: the slice's partial block goes to P.part and
// k_gather sums the slices.
template <int CT>
struct BigTile {
  static constexpr int TB = 4 * CT;        // packed 16-column tiles per block
  static constexpr int NP = 2 * CT;        // 32-column MFMA tiles per block
  static constexpr int LDO = 64 * CT + 4;  // output row stride in LDS (floats): rows 4 apart hit other banks
  static constexpr int RING = 2 * TB * 64;  // u32x4 words: two steps of TB weight fragments
  static constexpr int BYTES = (kMaxRows * LDO * 4 > RING * 16) ? kMaxRows * LDO * 4 : RING * 16;
};

// The pairs of a block's outputs staged in LDS (row r at sOut + r*LDO):
// pair idx = (row idx/(32CT), columns nb*64CT + 2*(idx%(32CT)) + {0,1}), as
// in for_pairs, so the epilogue bodies (and their lane groups) are the same.
template <int CT, class F>
__device__ __forceinline__ void for_pairs_lds(const GemmParams& P, int nb, const float* sOut, F&& f) {
  constexpr int PR = 32 * CT, LDO = BigTile<CT>::LDO;
  const int n = P.R * PR;
  for (int idx = threadIdx.x; idx < n; idx += 256) {
    const int r = idx / PR, pc = 2 * (idx % PR), c = nb * 64 * CT + pc;
    if (c < P.N) {
      const float2 v = *(const float2*)(sOut + r * LDO + pc);
      f(idx, r, c, v.x, v.y);
    }
  }
}

template <int EPI, int CT, int PD>
__global__ __launch_bounds__(256) void k_gemm_big(GemmParams P, int ksl) {
  constexpr int TB = BigTile<CT>::TB, NP = BigTile<CT>::NP;
  const int NB = (P.N + 64 * CT - 1) / (64 * CT), ns = P.nslices;
  const int id = blockIdx.x, xcd = id & 7, loc = id >> 3;
  const int nb = (loc / ns) * 8 + xcd, sl = loc % ns;
  if (nb >= NB) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nch = (P.R + 15) >> 4, KS = P.K >> 5, ks0 = sl * ksl, NT = (P.N + 15) >> 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[BigTile<CT>::BYTES];
  u32x4* ring = (u32x4*)smem;

  // This lane's A words (a chunk past nch repeats the last one; its rows are
  // never stored) and B word offsets within a ring slot, half h at +16h.
  const u32x4* af = (const u32x4*)P.Af;
  const int sub = (lane >> 4) & 1, g0 = (lane & 15) + 16 * (lane >> 5);
  const int awo = min(2 * wave + sub, nch - 1) * 64 + g0;
  const int bwo = sub * 64 + g0;
  // This lane's weight words: word tid + 256c of the block's TB fragments
  // (tiles past N load tile 0's; their outputs are never stored).
  const u32x4* wb[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int u = tid + 256 * c, tile = nb * TB + (u >> 6);
    wb[c] = (const u32x4*)P.W + (size_t)(tile < NT ? tile : 0) * KS * 64 + (u & 63);
  }
  u32x4 ra[PD][2], rb[PD][CT];
  auto issue_a = [&](int i, int ks) {
    const u32x4* a = af + (size_t)ks * nch * 64 + awo;
    ra[i][0] = a[0];
    ra[i][1] = a[32];
  };
  auto issue_b = [&](int i, int ks) {
#pragma unroll
    for (int c = 0; c < CT; ++c) rb[i][c] = __builtin_nontemporal_load(wb[c] + (size_t)ks * 64);
  };
#pragma unroll
  for (int i = 0; i < PD; ++i) {
    issue_b(i, ks0 + i);
    issue_a(i, ks0 + i);
  }

  f32x16 acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[p][v] = 0.0f;

  // ksl is a multiple of PD (the launcher checks): rounds of PD steps, every
  // round but the last issuing the next round's loads, so the loads in flight
  // at the loop's back edge are always the same and the waits count them
  // exactly.  A slot of a register ring is reloaded right after its last read.
  auto round = [&](int s, auto more) {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      u32x4* slot = ring + ((s + i) & 1) * (TB * 64);
#pragma unroll
      for (int c = 0; c < CT; ++c) slot[tid + 256 * c] = rb[i][c];
      if constexpr (decltype(more)::value) issue_b(i, ks0 + s + i + PD);
      __syncthreads();
      f16x8 bf[NP][2];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) bf[p][h] = __builtin_bit_cast(f16x8, slot[p * 128 + bwo + 32 * h]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ra[i][h]), bf[p][h], acc[p], 0, 0, 0);
      if constexpr (decltype(more)::value) issue_a(i, ks0 + s + i + PD);
    }
  };
  int s = 0;
  for (; s + PD < ksl; s += PD) round(s, std::true_type{});
  round(s, std::false_type{});

  // D: lane l value v is row 32w + 8*(v/4) + 4*(l/32) + v%4, column 32p + l%32.
  const int rb0 = 32 * wave + 4 * (lane >> 5), cl = lane & 31;
  if (ns > 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int col = nb * 64 * CT + 32 * p + cl;
      if (col < P.N)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = rb0 + 8 * (v >> 2) + (v & 3);
          if (r < P.R) P.part[((size_t)sl * P.R + r) * P.N + col] = acc[p][v];
        }
    }
    return;
  }
  constexpr int LDO = BigTile<CT>::LDO;
  float* sOut = (float*)smem;
  __syncthreads();  // the ring's last reads are done
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = rb0 + 8 * (v >> 2) + (v & 3);
      if (r < P.R) sOut[r * LDO + 32 * p + cl] = acc[p][v];
    }
  __syncthreads();
  if constexpr (EPI == EPI_QKV) {
    for_pairs_lds<CT>(P, nb, sOut, [&](int, int r, int c, float v0, float v1) { qkv_pair(P, r, c, v0, v1); });
  } else if constexpr (EPI == EPI_RESID) {
    const int NG = P.N >> 4;
    for_pairs_lds<CT>(P, nb, sOut, [&](int idx, int r, int c, float v0, float v1) {
      const float t = sum8(resid_pair(P, r, c, v0, v1));
      if ((idx & 7) == 0) P.ss_out[(size_t)r * NG + (c >> 4)] = t;
    });
  } else if constexpr (EPI == EPI_SWIGLU) {
    for_pairs_lds<CT>(P, nb, sOut, [&](int, int r, int c, float g, float u) { swiglu_prep_pair(P, r, c, g, u); });
  } else {
    const Sampling sm = load_sampling(P);
    for_pairs_lds<CT>(P, nb, sOut, [&](int idx, int r, int c, float v0, float v1) {
      unsigned long long k0, k1;
      lm_pair_keys(P, sm, r, c, v0, v1, P.rowinfo[2 * r], k0, k1);
      unsigned long long kk = k0 > k1 ? k0 : k1;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        const unsigned long long t = __shfl_xor(kk, o);
        kk = t > kk ? t : kk;
      }
      if ((idx & 31) == 0) atomicMax(&P.argkey[r], kk);
    });
    __syncthreads();  // sOut's last reads are done before lm_finish reuses it
    lm_finish(P, NB, sOut);
  }
}

// Sum of the NW K parts' partial tiles (part w at sAcc[(w*CT + ct)*64]) in
// groups of GP: the parts of each group in order, then the group sums in
// order, each sum from zero.  With GP = 1 or GP = NW this is the plain
// part-order sum of the split-K gather.
template <int NW, int GP, int CT>
__device__ __forceinline__ void group_sum(const f32x4* sAcc, int ct, int e0, float& v0, float& v1) {
#pragma clang fp contract(off)
  v0 = 0.0f;
  v1 = 0.0f;
#pragma unroll
  for (int gi = 0; gi < NW / GP; ++gi) {
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int p = 0; p < GP; ++p) {
      const float* t = (const float*)(sAcc + ((gi * GP + p) * CT + ct) * 64);
      a0 += t[e0];
      a1 += t[e0 + 4];
    }
    v0 += a0;
    v1 += a1;
  }
}

// ------------------------------------------------------- one-pass GEMM
//
// For R <= 16 rows.  A workgroup of NW waves walks column blocks of CT
// 16-column tiles, blockIdx.x, blockIdx.x + gridDim.x, ..., over the whole
// K; wave w owns the K part of steps [w*SPW, (w+1)*SPW).  The prologue loads
// the wave's A rows once, straight into the MFMA A-operand layout (lane l:
// row l%16, inputs 8*(l/16)..+8 of every step), applies the RMSNorm and
// rounds them to fp16 once; they then serve every block of the walk.
// Weights stream through NBUF register buffers: the fragments of the block
// NBUF walk steps ahead are issued as soon as the current block's MFMAs have
// read theirs, so NBUF blocks are in flight while one is reduced.  Per block each wave runs
// CT*SPW MFMA and leaves its partial tiles in LDS; the workgroup adds the
// parts in wave order and runs the epilogue.  No partial buffer, arrival
// counter or second pass, except for the LM head: its threads keep the
// largest argmax key of their (row, 16 columns) over the walk, each group
// makes one atomic max per row, and the last workgroup to arrive runs the
// accept stage.  The K parts, the MFMA order within a part and the
// order of the final additions are those of the split-K kernel with
// NK = SPW and NW slices, so the two agree bit for bit (the split-K kernel
// serves R > 16).
template <int EPI, int NW, int SPW, int CT, int NBUF, int GP>
__global__ __launch_bounds__(NW * 64) void k_mm(GemmParams P) {
  static_assert(NBUF == 1 || NBUF == 2, "one or two weight buffers");
  static_assert(NW % GP == 0, "parts form whole groups");
  constexpr int NT = NW * 64, KS = NW * SPW;
  constexpr bool NORM = EPI != EPI_RESID;
  constexpr int SSN = KS * 2;                  // RMSNorm partials per row (K = hidden, one per 16 columns)
  constexpr int SSI = (SSN + 15) / 16;         // of them per lane
  constexpr int GPT = (KS * 32 + NT - 1) / NT; // gain values per thread
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int s0 = wave * SPW;
  const int row = lane & 15, kg = lane >> 4;
  const int nblk = (P.N + 16 * CT - 1) / (16 * CT), G = (int)gridDim.x;

  __shared__ f32x4 sAcc[NW * CT * 64];
  __shared__ float sG[NORM ? KS * 32 : 1];
  __shared__ float sR[16];

  auto fetch = [&](u32x4 (&bw)[CT][SPW], int blk) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int tile = blk * CT + c;
      if (tile * 16 < P.N) {
        const u32x4* wp = (const u32x4*)P.W + ((size_t)tile * KS + s0) * 64 + lane;
#pragma unroll
        for (int j = 0; j < SPW; ++j) bw[c][j] = __builtin_nontemporal_load(wp + j * 64);
      } else {
#pragma unroll
        for (int j = 0; j < SPW; ++j) bw[c][j] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };

  // Issue order: the QKV rows' positions and blocks, the small RMSNorm
  // inputs, then the first block's weights, then A, so that waiting for the
  // former never waits for the weights.
  constexpr int PPT = (16 * 8 * CT + NT - 1) / NT;  // epilogue pairs per thread at 16 rows
  constexpr bool POS = EPI == EPI_QKV || EPI == EPI_LM;  // the rows' positions (RoPE, sampling)
  int qpos[POS ? PPT : 1], qblk[EPI == EPI_QKV ? PPT : 1];
  if constexpr (POS) {
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int r = (tid + it * NT) / (8 * CT), rc = r < P.R ? r : 0;
      qpos[it] = P.rowinfo[2 * rc];
      if constexpr (EPI == EPI_QKV) qblk[it] = P.rowinfo[2 * rc + 1];
    }
  }
  // QKV, one weight buffer: the RoPE (cos, sin) of a block's epilogue pairs
  // load with the block's weights (rope_cur), the next block's with its
  // refill (rope_nxt), so the epilogue waits for no load of its own
  constexpr bool RPF = EPI == EPI_QKV && NBUF == 1;
  float2 rope_cur[RPF ? PPT : 1], rope_nxt[RPF ? PPT : 1];
  auto fetch_rope = [&](float2 (&dst)[RPF ? PPT : 1], int blk_) {
    if constexpr (RPF) {
#pragma unroll
      for (int it = 0; it < PPT; ++it) {
        const int pr = tid + it * NT, rem = pr % (8 * CT);
        const int col = (blk_ * CT + (rem >> 3)) * 16 + 2 * (rem & 7);
        dst[it] = pr < P.R * 8 * CT && col < P.N ? rope_cs(P, col, qpos[it]) : make_float2(0.0f, 0.0f);
      }
    }
  };
  Sampling sm = {0.0f, 0u, 0u};
  if constexpr (EPI == EPI_LM) sm = load_sampling(P);
  float gv[NORM ? GPT : 1], sv[NORM ? SSI : 1];
  const int ss_r = tid >> 4, ss_j = tid & 15;
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int e = tid + i * NT;
      gv[i] = e < KS * 32 ? P.gain[e] : 0.0f;
    }
    if constexpr (NT >= 256) {
#pragma unroll
      for (int i = 0; i < SSI; ++i) {
        const int q = ss_j + 16 * i;
        sv[i] = (tid < 256 && ss_r < P.R && q < SSN) ? P.ss[(size_t)ss_r * SSN + q] : 0.0f;
      }
    }
  }
  // LM head: a pair of each thread's (row, 16 columns) group keeps the
  // largest argmax key over the walk; one atomic per group at the end.
  unsigned long long kmax[EPI == EPI_LM ? PPT : 1];
#pragma unroll
  for (int it = 0; it < (EPI == EPI_LM ? PPT : 1); ++it) kmax[it] = 0ull;
  u32x4 b0[CT][SPW], b1[NBUF == 2 ? CT : 1][NBUF == 2 ? SPW : 1];
  int blk = blockIdx.x;
  fetch(b0, blk);
  fetch_rope(rope_cur, blk);
  f32x4 a[SPW][2];
  if (row < P.R) {
    const f32x4* ap = (const f32x4*)(P.A + (size_t)row * P.lda + s0 * 32 + kg * 8);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      a[j][0] = ap[j * 8];
      a[j][1] = ap[j * 8 + 1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPW; ++j) a[j][0] = a[j][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  }
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int e = tid + i * NT;
      if (e < KS * 32) sG[e] = gv[i];
    }
    if constexpr (NT >= 256) {
      if (tid < 256) {
        float acc = 0.0f;  // the order of rstd16: partials j, j + 16, ... then the xor tree
#pragma unroll
        for (int i = 0; i < SSI; ++i) acc += sv[i];
        const float rs = rstd_finish(acc, P.inv_dim, P.eps);
        if (ss_j == 0) sR[ss_r] = ss_r < P.R ? rs : 0.0f;
      }
    } else {
      for (int t = tid; t < 256; t += NT) {
        const int r = t >> 4, j = t & 15;
        const float rs = rstd16(P.ss, SSN, r, P.R, j, P.inv_dim, P.eps);
        if (j == 0) sR[r] = r < P.R ? rs : 0.0f;
      }
    }
    __syncthreads();
  }
  if constexpr (NORM) {  // normalised in place
    const float rs = sR[row];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const float* g = sG + (s0 + j) * 32 + kg * 8;
      a[j][0] = (f32x4){(a[j][0].x * rs) * g[0], (a[j][0].y * rs) * g[1], (a[j][0].z * rs) * g[2], (a[j][0].w * rs) * g[3]};
      a[j][1] = (f32x4){(a[j][1].x * rs) * g[4], (a[j][1].y * rs) * g[5], (a[j][1].z * rs) * g[6], (a[j][1].w * rs) * g[7]};
    }
  }
  // the A operand of every block: fp16, rounded once
  f16x8 a16[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const float v[8] = {a[j][0].x, a[j][0].y, a[j][0].z, a[j][0].w, a[j][1].x, a[j][1].y, a[j][1].z, a[j][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) a16[j][e] = (_Float16)v[e];
  }

  // One block: MFMA on bw, then (bw free) issue the block NBUF steps ahead
  // into it, then the reduction and the epilogue.
  auto pass = [&](u32x4 (&bw)[CT][SPW], int cur, int refill) {
    f32x4 acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int c = 0; c < CT; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a16[j], __builtin_bit_cast(f16x8, bw[c][j]), acc[c], 0, 0, 0);
    if (refill < nblk) {
      fetch(bw, refill);
      fetch_rope(rope_nxt, refill);
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) sAcc[(wave * CT + c) * 64 + lane] = acc[c];
    __syncthreads();
    // Column pairs: p = (row * CT + tile) * 8 + pair; an aligned group of 8
    // pairs is 16 columns of one row (the RMSNorm partial-sum group).  The
    // D layout keeps element (row r, column cc) of a tile in component r%4
    // of lane 16*(r/4) + cc.
    const int npairs = P.R * 8 * CT;
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int p = tid + it * NT;
      if (p < npairs) {
        const int r = p / (8 * CT), rem = p - r * (8 * CT), ct = rem >> 3, pp = rem & 7;
        const int col = (cur * CT + ct) * 16 + 2 * pp;
        const int e0 = ((r >> 2) * 16 + 2 * pp) * 4 + (r & 3);
        float v0, v1;
        group_sum<NW, GP, CT>(sAcc, ct, e0, v0, v1);
        if (col < P.N) {
          if constexpr (RPF) {
            qkv_pair_cs(P, r, col, v0, v1, qpos[it], qblk[it], rope_cur[it]);
          } else if constexpr (EPI == EPI_QKV) {
            qkv_pair_at(P, r, col, v0, v1, qpos[it], qblk[it]);
          } else if constexpr (EPI == EPI_RESID) {
            const float t = sum8(resid_pair(P, r, col, v0, v1));
            if ((p & 7) == 0) P.ss_out[(size_t)r * (P.N >> 4) + (col >> 4)] = t;
          } else if constexpr (EPI == EPI_SWIGLU) {
            swiglu_pair(P, r, col, v0, v1);
          } else {
            unsigned long long k0, k1;
            lm_pair_keys(P, sm, r, col, v0, v1, qpos[it], k0, k1);
            const unsigned long long k = k0 > k1 ? k0 : k1;
            kmax[it] = k > kmax[it] ? k : kmax[it];
          }
        }
      }
    }
    __syncthreads();  // sAcc is rewritten by the next block
    if constexpr (RPF) {
#pragma unroll
      for (int it = 0; it < PPT; ++it) rope_cur[it] = rope_nxt[it];
    }
  };

  // blocks blk, blk + G, ...; with two buffers b0 and b1 alternate without
  // register copies
  if constexpr (NBUF == 2) {
    if (blk + G < nblk) fetch(b1, blk + G);
    while (blk < nblk) {
      pass(b0, blk, blk + 2 * G);
      blk += G;
      if (blk >= nblk) break;
      pass(b1, blk, blk + 2 * G);
      blk += G;
    }
  } else {
    for (; blk < nblk; blk += G) pass(b0, blk, blk + G);
  }
  if constexpr (EPI == EPI_LM) {
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      unsigned long long k = kmax[it];
#pragma unroll
      for (int o = 4; o >= 1; o >>= 1) {
        const unsigned long long t = __shfl_xor(k, o);
        k = t > k ? t : k;
      }
      const int p = tid + it * NT;
      if (p < P.R * 8 * CT && (p & 7) == 0) atomicMax(&P.argkey[p / (8 * CT)], k);
    }
    lm_finish(P, G, (float*)sAcc);
  }
}

// The same arithmetic for one 16-column tile per workgroup (grid = tiles)
// with the wave's SPW steps loaded and multiplied in PH phases of up to
// SPP steps: phase p+1's weights and A rows are issued once phase p's MFMAs
// have read theirs, so a K part too long for the registers still runs in
// one pass (each phase adds one memory latency, not a second kernel).
template <int EPI, int NW, int SPW, int PH, int GP, bool H16 = false>
__global__ __launch_bounds__(NW * 64) void k_mm1(GemmParams P) {
  static_assert(NW % GP == 0, "parts form whole groups");
  static_assert(!H16 || EPI == EPI_RESID, "fp16 A rows carry no RMSNorm");
  constexpr int NT = NW * 64, KS = NW * SPW, SPP = (SPW + PH - 1) / PH;
  constexpr bool NORM = EPI != EPI_RESID;
  constexpr int SSN = KS * 2, SSI = (SSN + 15) / 16, GPT = (KS * 32 + NT - 1) / NT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = blockIdx.x, s0 = wave * SPW;
  const int row = lane & 15, kg = lane >> 4;

  __shared__ f32x4 sAcc[NW * 64];
  __shared__ float sG[NORM ? KS * 32 : 1];
  __shared__ float sR[16];

  float gv[NORM ? GPT : 1], sv[NORM ? SSI : 1];
  const int ss_r = tid >> 4, ss_j = tid & 15;
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int e = tid + i * NT;
      gv[i] = e < KS * 32 ? P.gain[e] : 0.0f;
    }
    if constexpr (NT >= 256) {
#pragma unroll
      for (int i = 0; i < SSI; ++i) {
        const int q = ss_j + 16 * i;
        sv[i] = (tid < 256 && ss_r < P.R && q < SSN) ? P.ss[(size_t)ss_r * SSN + q] : 0.0f;
      }
    }
  }
  const u32x4* wp = (const u32x4*)P.W + ((size_t)tile * KS + s0) * 64 + lane;
  const f32x4* ap = (const f32x4*)(P.A + (size_t)row * P.lda + s0 * 32 + kg * 8);
  const u32x4* ap16 = nullptr;
  if constexpr (H16) ap16 = (const u32x4*)(P.A16 + (size_t)row * P.lda + s0 * 32 + kg * 8);
  const bool arow = row < P.R;
  static_assert(NT >= 128, "one epilogue pair per thread at 16 rows");
  const int npairs = P.R * 8, er = tid >> 3, epp = tid & 7, ecol = tile * 16 + 2 * epp;
  // residual epilogue: this thread's pair of x, issued before everything else
  float2 xv = make_float2(0.0f, 0.0f);
  if constexpr (EPI == EPI_RESID)
    if (tid < npairs) xv = *(const float2*)(P.x + (size_t)er * P.N + ecol);
  u32x4 b[SPP];
  f32x4 a[H16 ? 1 : SPP][2];
  u32x4 ah[H16 ? SPP : 1];
#define SPECV_MM1_LOAD(J0)                                                  \
  _Pragma("unroll") for (int j = 0; j < SPP; ++j) if ((J0) + j < SPW) b[j] = \
      __builtin_nontemporal_load(wp + ((J0) + j) * 64);                       \
  _Pragma("unroll") for (int j = 0; j < SPP; ++j) {                          \
    if constexpr (H16) {                                                     \
      ah[j] = (arow && (J0) + j < SPW) ? ap16[((J0) + j) * 4] : (u32x4){0u, 0u, 0u, 0u}; \
    } else if (arow && (J0) + j < SPW) {                                     \
      a[j][0] = ap[((J0) + j) * 8];                                          \
      a[j][1] = ap[((J0) + j) * 8 + 1];                                      \
    } else {                                                                 \
      a[j][0] = a[j][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};                   \
    }                                                                        \
  }
  SPECV_MM1_LOAD(0)
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int e = tid + i * NT;
      if (e < KS * 32) sG[e] = gv[i];
    }
    if constexpr (NT >= 256) {
      if (tid < 256) {
        float acc = 0.0f;  // the order of rstd16
#pragma unroll
        for (int i = 0; i < SSI; ++i) acc += sv[i];
        const float rs = rstd_finish(acc, P.inv_dim, P.eps);
        if (ss_j == 0) sR[ss_r] = ss_r < P.R ? rs : 0.0f;
      }
    } else {
      for (int t = tid; t < 256; t += NT) {
        const int r = t >> 4, j = t & 15;
        const float rs = rstd16(P.ss, SSN, r, P.R, j, P.inv_dim, P.eps);
        if (j == 0) sR[r] = r < P.R ? rs : 0.0f;
      }
    }
    __syncthreads();
  }
  const float rs = NORM ? sR[row] : 1.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ph = 0; ph < PH; ++ph) {
    if (ph > 0) {
      SPECV_MM1_LOAD(ph * SPP)
    }
#pragma unroll
    for (int j = 0; j < SPP; ++j) {
      if (ph * SPP + j < SPW) {
        f16x8 h;
        if constexpr (H16) {
          h = __builtin_bit_cast(f16x8, ah[j]);
        } else {
          float v[8] = {a[j][0].x, a[j][0].y, a[j][0].z, a[j][0].w, a[j][1].x, a[j][1].y, a[j][1].z, a[j][1].w};
          if constexpr (NORM) {
            const float* g = sG + (s0 + ph * SPP + j) * 32 + kg * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (v[e] * rs) * g[e];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[e];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(h, __builtin_bit_cast(f16x8, b[j]), acc, 0, 0, 0);
      }
    }
  }
#undef SPECV_MM1_LOAD
  sAcc[wave * 64 + lane] = acc;
  __syncthreads();
  if (tid < npairs) {
    const int e0 = ((er >> 2) * 16 + 2 * epp) * 4 + (er & 3);
    float v0, v1;
    group_sum<NW, GP, 1>(sAcc, 0, e0, v0, v1);
    if constexpr (EPI == EPI_QKV) {
      qkv_pair(P, er, ecol, v0, v1);
    } else if constexpr (EPI == EPI_RESID) {
      const float t = sum8(resid_pair_x(P, er, ecol, v0, v1, xv));
      if (epp == 0) P.ss_out[(size_t)er * (P.N >> 4) + (ecol >> 4)] = t;
    } else {
      swiglu_pair(P, er, ecol, v0, v1);
    }
  }
}

// The same arithmetic as k_mm1 (one tile per workgroup, NW K parts of SPW
// steps, parts summed in order) for at most RL rows with A staged in LDS:
// up to eight rows of the whole A as fp16 fit the LDS even at K = 9728
// (155,648 bytes), so each wave keeps all of its SPW weight fragments in
// flight at once, however long its K part (the residual epilogue only).
// The A rows are loaded first, the weights second, so the staging waits for
// the A rows alone and runs while the weights stream.
template <int NW, int SPW, int RL, bool H16 = false>
__global__ __launch_bounds__(NW * 64) void k_mm1l(GemmParams P) {
  constexpr int NT = NW * 64, KS = NW * SPW;
  constexpr int UNITS = RL * KS * 4, UPT = (UNITS + NT - 1) / NT;  // (row, step, lane group) units of 8 inputs
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = blockIdx.x, s0 = wave * SPW;
  const int row = lane & 15, kg = lane >> 4;
  // this thread's pair of x for the residual epilogue (8 R <= 32 pairs), issued first
  static_assert(NT >= 8 * RL, "one epilogue pair per thread");
  const int npairs = P.R * 8, er = tid >> 3, epp = tid & 7, ecol = tile * 16 + 2 * epp;
  float2 xv = make_float2(0.0f, 0.0f);
  if (tid < npairs) xv = *(const float2*)(P.x + (size_t)er * P.N + ecol);

  __shared__ u32x4 sA[KS * 4 * RL];  // [step][lane group][row], fp16; then the partial tiles
  static_assert(NW * 64 <= KS * 4 * RL, "the partial tiles fit the A buffer");
  f32x4* sAcc = (f32x4*)sA;

  // A staged in NB batches of UPB units per thread, the first batch's loads
  // ahead of the weights (at eight rows of K = 9728 a single batch would hold
  // 80 registers of A beside the 76 of the weights)
  // (fp16 rows: half the registers per unit, so up to 12 units in one batch)
  constexpr int NB = H16 ? (UPT > 12 ? (UPT + 7) / 8 : 1) : (UPT > 6 ? (UPT + 3) / 4 : 1);
  constexpr int UPB = (UPT + NB - 1) / NB;
  f32x4 pa[H16 ? 1 : UPB][2];
  u32x4 ph[H16 ? UPB : 1];
  auto load_a = [&](int bt) {
#pragma unroll
    for (int i = 0; i < UPB; ++i) {
      const int u = tid + (bt * UPB + i) * NT;
      const int r = u % RL, g = (u / RL) & 3, j = u / (RL * 4);
      const bool ok = u < UNITS && r < P.R;
      const size_t off = (size_t)(ok ? r : 0) * P.lda + (size_t)(ok ? j : 0) * 32 + g * 8;
      if constexpr (H16) {
        ph[i] = *(const u32x4*)(P.A16 + off);
      } else {
        const f32x4* src = (const f32x4*)(P.A + off);
        pa[i][0] = src[0];
        pa[i][1] = src[1];
      }
    }
  };
  auto stage_a = [&](int bt) {
#pragma unroll
    for (int i = 0; i < UPB; ++i) {
      const int u = tid + (bt * UPB + i) * NT;
      if (u < UNITS) {
        const int r = u % RL, g = (u / RL) & 3, j = u / (RL * 4);
        const bool ok = r < P.R;
        u32x4 hv;
        if constexpr (H16) {
          hv = ok ? ph[i] : (u32x4){0u, 0u, 0u, 0u};
        } else {
          float v[8] = {pa[i][0].x, pa[i][0].y, pa[i][0].z, pa[i][0].w, pa[i][1].x, pa[i][1].y, pa[i][1].z, pa[i][1].w};
          f16x8 h;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (_Float16)(ok ? v[e] : 0.0f);
          hv = __builtin_bit_cast(u32x4, h);
        }
        sA[(j * 4 + g) * RL + r] = hv;
      }
    }
  };
  load_a(0);
  const u32x4* wp = (const u32x4*)P.W + ((size_t)tile * KS + s0) * 64 + lane;
  u32x4 b[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) b[j] = __builtin_nontemporal_load(wp + j * 64);
  stage_a(0);
#pragma unroll
  for (int bt = 1; bt < NB; ++bt) {
    load_a(bt);
    stage_a(bt);
  }
  __syncthreads();
  const bool rok = row < P.R && row < RL;
  const int rc = row < RL ? row : RL - 1;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 h = sA[((s0 + j) * 4 + kg) * RL + rc];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, rok ? h : z),
                                                 __builtin_bit_cast(f16x8, b[j]), acc, 0, 0, 0);
  }
  __syncthreads();  // every wave is done with A
  sAcc[wave * 64 + lane] = acc;
  __syncthreads();
  if (tid < npairs) {
    const int e0 = ((er >> 2) * 16 + 2 * epp) * 4 + (er & 3);
    float v0, v1;
    group_sum<NW, 1, 1>(sAcc, 0, e0, v0, v1);
    const float t = sum8(resid_pair_x(P, er, ecol, v0, v1, xv));
    if (epp == 0) P.ss_out[(size_t)er * (P.N >> 4) + (ecol >> 4)] = t;
  }
}

// The int4 one-pass GEMM for at most eight rows (K = hidden or n_q * hd),
// activations staged in LDS (RL = 4 or 8 staged rows, the same arithmetic):
// every workgroup stages the whole normalised activation once in LDS as fp16
// in the MFMA A-operand order ([step][lane group][row]),
// then walks blocks of CT 16-column tiles (blockIdx.x, + gridDim.x, ...),
// reading each A fragment from LDS once for the CT tiles.  Wave w owns
// the K part of groups [w*GPW, (w+1)*GPW) of 128 inputs: per group the four
// steps' MFMAs on the exact integer weights, then one fused multiply-add by
// the column's group scale -- the arithmetic of the int4 split-K kernel with
// 4*GPW-step slices -- and the parts are added in wave order, so both agree
// bit for bit (each tile's sums keep their order whatever CT is).  The next
// block's fragments are issued as soon as the MFMAs have read the current
// ones.
template <int EPI, int NW, int GPW, int CT, int RL, bool H16 = false>
__global__ __launch_bounds__(NW * 64) void k_mmq(GemmParams P) {
  static_assert(!H16 || EPI == EPI_RESID, "fp16 A rows carry no RMSNorm");
  constexpr int NT = NW * 64, KG = NW * GPW, KS = KG * 4;
  constexpr bool NORM = EPI != EPI_RESID;
  constexpr int UNITS = RL * KS * 4, UPT = (UNITS + NT - 1) / NT;  // (row, step, lane group) units of 8 inputs
  constexpr int PPT = (RL * 8 * CT + NT - 1) / NT;                 // epilogue pairs per thread
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g0 = wave * GPW, row = lane & 15, kg = lane >> 4;
  const int ntile = P.N >> 4, nblk = (ntile + CT - 1) / CT, G = (int)gridDim.x;

  __shared__ u32x4 sA[KS * 4 * RL];  // [step][lane group][row], fp16
  __shared__ f32x4 sAcc[NW * 64 * CT];
  __shared__ float sR[RL];

  // Issue order: the QKV rows' positions, A and the gains (needed first),
  // then the first tile's weights and scales, then the RMSNorm row
  // statistics (one wave).
  constexpr bool POS = EPI == EPI_QKV || EPI == EPI_LM;  // the rows' positions (RoPE, sampling)
  int qpos[POS ? PPT : 1], qblk[EPI == EPI_QKV ? PPT : 1];
  if constexpr (POS) {
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int r = (tid + it * NT) / (8 * CT), rc = r < P.R ? r : 0;
      qpos[it] = P.rowinfo[2 * rc];
      if constexpr (EPI == EPI_QKV) qblk[it] = P.rowinfo[2 * rc + 1];
    }
  }
  Sampling sm = {0.0f, 0u, 0u};
  if constexpr (EPI == EPI_LM) sm = load_sampling(P);
  f32x4 pa[H16 ? 1 : UPT][2], pg[NORM ? UPT : 1][2];
  u32x4 ph[H16 ? UPT : 1];  // or the rows already rounded to fp16
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    const int r = u % RL, g = (u / RL) & 3, j = u / (RL * 4);
    const bool ok = u < UNITS && r < P.R;
    const int jc = u < UNITS ? j : 0;
    const size_t off = (size_t)(ok ? r : 0) * P.lda + (size_t)(ok ? j : 0) * 32 + g * 8;
    if constexpr (H16) {
      ph[i] = *(const u32x4*)(P.A16 + off);
    } else {
      const f32x4* src = (const f32x4*)(P.A + off);
      pa[i][0] = src[0];
      pa[i][1] = src[1];
    }
    if constexpr (NORM) {
      const f32x4* gsrc = (const f32x4*)(P.gain + (size_t)jc * 32 + g * 8);
      pg[i][0] = gsrc[0];
      pg[i][1] = gsrc[1];
    }
  }
  // one weight buffer (CT tiles): the next block is issued once the MFMAs
  // have read it; a block's tiles past the last (odd tile counts) reload the
  // last tile, and their columns are not stored
  u32x4 b0[CT][GPW];
  uint32_t s0[CT][GPW];  // raw bf16 scale bits, converted at use (no wait on arrival)
  auto fetch = [&](u32x4 (&bw)[CT][GPW], uint32_t (&sw)[CT][GPW], int blk_) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int tile = min(blk_ * CT + c, ntile - 1);
      const u32x4* wp = (const u32x4*)P.W + ((size_t)tile * KG + g0) * 64 + lane;
      const uint16_t* sp = P.scales + ((size_t)tile * 16 + (lane & 15)) * KG + g0;
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        bw[c][gi] = __builtin_nontemporal_load(wp + gi * 64);
        sw[c][gi] = sp[gi];
      }
    }
  };
  int blk = blockIdx.x;
  if (blk < nblk) fetch(b0, s0, blk);
  if constexpr (NORM) {  // rstd of the rows (rstd16, 16 lanes per row, whole waves), after every load is out
    for (int t = tid; t < 16 * RL; t += NT) {
      const float rs = rstd16(P.ss, P.ss_n, t >> 4, P.R, t & 15, P.inv_dim, P.eps);
      if ((t & 15) == 0) sR[t >> 4] = (t >> 4) < P.R ? rs : 0.0f;
    }
    __syncthreads();
  }
  // A into LDS as fp16 (the int4 split-K kernel's conversion)
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u < UNITS) {
      const int r = u % RL, g = (u / RL) & 3, j = u / (RL * 4);
      if constexpr (H16) {
        sA[(j * 4 + g) * RL + r] = r < P.R ? ph[i] : (u32x4){0u, 0u, 0u, 0u};
      } else {
        float v[8] = {pa[i][0].x, pa[i][0].y, pa[i][0].z, pa[i][0].w, pa[i][1].x, pa[i][1].y, pa[i][1].z, pa[i][1].w};
        if (r >= P.R) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
        if constexpr (NORM) {
          const float sc = r < P.R ? sR[r] : 0.0f;
          const float gv[8] = {pg[i][0].x, pg[i][0].y, pg[i][0].z, pg[i][0].w, pg[i][1].x, pg[i][1].y, pg[i][1].z, pg[i][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (v[e] * sc) * gv[e];
        }
        f16x8 hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) hi[e] = (_Float16)v[e];
        sA[(j * 4 + g) * RL + r] = __builtin_bit_cast(u32x4, hi);
      }
    }
  }
  __syncthreads();
  // Lanes of rows past RL read row RL - 1 (rows R..RL-1 were staged as
  // zeros): an MFMA output row depends on its own A row alone, and rows past
  // R are never stored, so no per-lane select is needed on the A fragments.
  const int rc = row < RL ? row : RL - 1;
  unsigned long long kmax[EPI == EPI_LM ? PPT : 1];
#pragma unroll
  for (int it = 0; it < (EPI == EPI_LM ? PPT : 1); ++it) kmax[it] = 0ull;

  // One block of CT tiles on the weights in bw, then (bw free) the block
  // refill into it, then the reduction and the epilogue.
  auto pass = [&](u32x4 (&bw)[CT][GPW], uint32_t (&sw)[CT][GPW], int cur, int refill) {
    f32x4 acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      f32x4 t[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) t[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int j = (g0 + gi) * 4 + d;
        const f16x8 ah = __builtin_bit_cast(f16x8, sA[(j * 4 + kg) * RL + rc]);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const f16x8 bq = dequant8_ao(bw[c][gi][d]);
          t[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, t[c], 0, 0, 0);
        }
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const float sc = bf16_bits_to_f32((uint16_t)sw[c][gi]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] = __builtin_fmaf(t[c][i], sc, acc[c][i]);
      }
    }
    if (refill < nblk) fetch(bw, sw, refill);
#pragma unroll
    for (int c = 0; c < CT; ++c) sAcc[(wave * CT + c) * 64 + lane] = acc[c];
    __syncthreads();
    // p = (row * CT + tile) * 8 + pair: an aligned group of 8 pairs is 16
    // columns of one row
    const int npairs = P.R * 8 * CT;
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int p = tid + it * NT;
      const int r = p / (8 * CT), rem = p - r * (8 * CT), ct = rem >> 3, pp = rem & 7;
      const int col = (cur * CT + ct) * 16 + 2 * pp;
      if (p < npairs && col < P.N) {
        const int e0 = ((r >> 2) * 16 + 2 * pp) * 4 + (r & 3);
        float v0, v1;
        group_sum<NW, 1, CT>(sAcc, ct, e0, v0, v1);
        if constexpr (EPI == EPI_QKV) {
          qkv_pair_at(P, r, col, v0, v1, qpos[it], qblk[it]);
        } else if constexpr (EPI == EPI_RESID) {
          const float s8 = sum8(resid_pair(P, r, col, v0, v1));
          if ((p & 7) == 0) P.ss_out[(size_t)r * (P.N >> 4) + (col >> 4)] = s8;
        } else if constexpr (EPI == EPI_SWIGLU) {
          swiglu_pair(P, r, col, v0, v1);
        } else {
          unsigned long long k0, k1;
          lm_pair_keys(P, sm, r, col, v0, v1, qpos[it], k0, k1);
          const unsigned long long k = k0 > k1 ? k0 : k1;
          kmax[it] = k > kmax[it] ? k : kmax[it];
        }
      }
    }
    __syncthreads();  // sAcc is rewritten by the next tile
  };
  for (; blk < nblk; blk += G) pass(b0, s0, blk, blk + G);
  if constexpr (EPI == EPI_LM) {
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      unsigned long long k = kmax[it];
#pragma unroll
      for (int o = 4; o >= 1; o >>= 1) {
        const unsigned long long t = __shfl_xor(k, o);
        k = t > k ? t : k;
      }
      const int p = tid + it * NT;
      if (p < P.R * 8 * CT && (p & 7) == 0) atomicMax(&P.argkey[p / (8 * CT)], k);
    }
    lm_finish(P, G, (float*)sAcc);
  }
}

// The int4 one-pass GEMM for up to 16 rows, activations in registers.  A
// workgroup of NW waves owns one K part of KG = NW*GPW groups of 128 inputs
// (part kp of the K / (KG*128) parts: workgroup blockIdx.x takes part
// blockIdx.x % parts and walks the column blocks blockIdx.x / parts,
// + gridDim.x / parts, ...).  Every lane loads its own A values once, straight
// into the MFMA A-operand layout (lane l: row l%16, inputs 8*(l/16)..+8 of
// each of the wave's 4*GPW steps), applies the RMSNorm (the gains staged in
// LDS) and keeps them as fp16 for the whole walk, so the row count
// costs no LDS and no weight is read twice: rows up to 16 run the same
// instructions as one row.  Per tile and group the four steps' MFMAs on the
// exact integer weights, then one fused multiply-add by the column's group
// scale; the wave parts are added in wave order.  With one K part the
// epilogue follows at once; with several (O, down) each part's tile goes to
// the split buffer, and after the walk the last part of each tile to arrive
// (an arrival counter per block) adds the parts in part order and runs the
// residual epilogue.  Every sum's order depends on the shape of the GEMM
// alone, never on R, so an S-row forward equals S one-row forwards bit for bit.
constexpr int kMmqrMaxParts = 8;  // K parts of the register kernel's plans (host-checked)

template <int EPI, int NW, int GPW, int CT, bool H16 = false>
__global__ __launch_bounds__(NW * 64) void k_mmqr(GemmParams P) {
  static_assert(!H16 || EPI == EPI_RESID, "fp16 A rows carry no RMSNorm");
  constexpr int NT = NW * 64, KG = NW * GPW, ST = GPW * 4;
  constexpr bool NORM = EPI != EPI_RESID;
  constexpr int PPT = (16 * 8 * CT + NT - 1) / NT;  // epilogue pairs per thread
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = lane & 15, kg = lane >> 4;
  const int parts = P.nslices;  // K parts (host-checked: K = parts * KG * 128, gridDim.x % parts == 0)
  const int kp = (int)blockIdx.x % parts, wg = (int)blockIdx.x / parts, GW = (int)gridDim.x / parts;
  const int KGT = P.K >> 7;            // groups over the whole K
  const int g0 = kp * KG + wave * GPW; // the wave's first group
  const int ntile = P.N >> 4, nblk = (ntile + CT - 1) / CT;

  __shared__ float sG[NORM ? KG * 128 : 1];
  __shared__ f32x4 sAcc[NW * 64 * CT];
  __shared__ float sR[16];
  __shared__ int sLast;
  __shared__ int sDone[64];  // residual parts: blocks this workgroup completes, per round

  constexpr bool POS = EPI == EPI_QKV || EPI == EPI_LM;
  int qpos[POS ? PPT : 1], qblk[EPI == EPI_QKV ? PPT : 1];
  if constexpr (POS) {
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int r = (tid + it * NT) / (8 * CT), rc = r < P.R ? r : 0;
      qpos[it] = P.rowinfo[2 * rc];
      if constexpr (EPI == EPI_QKV) qblk[it] = P.rowinfo[2 * rc + 1];
    }
  }
  Sampling sm = {0.0f, 0u, 0u};
  if constexpr (EPI == EPI_LM) sm = load_sampling(P);
  // the lane's A values: 8 per step, rows past R are zeros (or the rows
  // already rounded to fp16)
  float a[H16 ? 1 : ST][8];
  u32x4 a16[H16 ? ST : 1];
  if constexpr (H16) {
    const bool live = row < P.R;
    const _Float16* src = P.A16 + (size_t)(live ? row : 0) * P.lda + (size_t)g0 * 128 + kg * 8;
#pragma unroll
    for (int j = 0; j < ST; ++j) a16[j] = live ? *(const u32x4*)(src + j * 32) : (u32x4){0u, 0u, 0u, 0u};
  } else {
    const bool live = row < P.R;
    const float* src = P.A + (size_t)(live ? row : 0) * P.lda + (size_t)g0 * 128 + kg * 8;
#pragma unroll
    for (int j = 0; j < ST; ++j) {
      const f32x4 x0 = live ? *(const f32x4*)(src + j * 32) : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 x1 = live ? *(const f32x4*)(src + j * 32 + 4) : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      a[j][0] = x0.x; a[j][1] = x0.y; a[j][2] = x0.z; a[j][3] = x0.w;
      a[j][4] = x1.x; a[j][5] = x1.y; a[j][6] = x1.z; a[j][7] = x1.w;
    }
  }
  if constexpr (NORM) {  // the workgroup's gains, coalesced
    const f32x4* gsrc = (const f32x4*)(P.gain + (size_t)kp * KG * 128);
    for (int i = tid; i < KG * 32; i += NT) ((f32x4*)sG)[i] = gsrc[i];
  }
  u32x4 b0[CT][GPW];
  uint32_t s0[CT][GPW];  // raw bf16 scale bits, converted at use
  auto fetch = [&](u32x4 (&bw)[CT][GPW], uint32_t (&sw)[CT][GPW], int blk_) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int tile = min(blk_ * CT + c, ntile - 1);
      const u32x4* wp = (const u32x4*)P.W + ((size_t)tile * KGT + g0) * 64 + lane;
      const uint16_t* sp = P.scales + ((size_t)tile * 16 + (lane & 15)) * KGT + g0;
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        bw[c][gi] = __builtin_nontemporal_load(wp + gi * 64);
        sw[c][gi] = sp[gi];
      }
    }
  };
  int blk = wg;
  if (blk < nblk) fetch(b0, s0, blk);
  if constexpr (NORM) {  // rstd of the 16 rows (16 lanes per row, whole waves), after every load is out
    for (int t = tid; t < 256; t += NT) {
      const float rs = rstd16(P.ss, P.ss_n, t >> 4, P.R, t & 15, P.inv_dim, P.eps);
      if ((t & 15) == 0) sR[t >> 4] = (t >> 4) < P.R ? rs : 0.0f;
    }
  }
  __syncthreads();
  // normalise and round to fp16, in place
  f16x8 ah[ST];
  if constexpr (H16) {
#pragma unroll
    for (int j = 0; j < ST; ++j) ah[j] = __builtin_bit_cast(f16x8, a16[j]);
  } else {
    const float sc = NORM ? sR[row] : 1.0f;
#pragma unroll
    for (int j = 0; j < ST; ++j) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = a[j][e];
      if constexpr (NORM) {
        const f32x4 g0v = *(const f32x4*)(sG + (wave * GPW * 4 + j) * 32 + kg * 8);
        const f32x4 g1v = *(const f32x4*)(sG + (wave * GPW * 4 + j) * 32 + kg * 8 + 4);
        const float gv[8] = {g0v.x, g0v.y, g0v.z, g0v.w, g1v.x, g1v.y, g1v.z, g1v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (v[e] * sc) * gv[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ah[j][e] = (_Float16)v[e];
    }
  }
  unsigned long long kmax[EPI == EPI_LM ? PPT : 1];
#pragma unroll
  for (int it = 0; it < (EPI == EPI_LM ? PPT : 1); ++it) kmax[it] = 0ull;

  auto pass = [&](u32x4 (&bw)[CT][GPW], uint32_t (&sw)[CT][GPW], int cur, int refill) {
    f32x4 acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      f32x4 t[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) t[c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const f16x8 bq = dequant8_ao(bw[c][gi][d]);
          t[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[gi * 4 + d], bq, t[c], 0, 0, 0);
        }
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const float sc = bf16_bits_to_f32((uint16_t)sw[c][gi]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] = __builtin_fmaf(t[c][i], sc, acc[c][i]);
      }
    }
    if (refill < nblk) fetch(bw, sw, refill);
#pragma unroll
    for (int c = 0; c < CT; ++c) sAcc[(wave * CT + c) * 64 + lane] = acc[c];
    __syncthreads();
    // p = (row * CT + tile) * 8 + pair: an aligned group of 8 pairs is 16
    // columns of one row
    const int npairs = P.R * 8 * CT;
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int p = tid + it * NT;
      const int r = p / (8 * CT), rem = p - r * (8 * CT), ct = rem >> 3, pp = rem & 7;
      const int col = (cur * CT + ct) * 16 + 2 * pp;
      if (p < npairs && col < P.N) {
        const int e0 = ((r >> 2) * 16 + 2 * pp) * 4 + (r & 3);
        float v0, v1;
        group_sum<NW, 1, CT>(sAcc, ct, e0, v0, v1);
        if constexpr (EPI == EPI_QKV) {
          qkv_pair_at(P, r, col, v0, v1, qpos[it], qblk[it]);
        } else if constexpr (EPI == EPI_RESID) {
          if (parts > 1) {
            st_dev2(P.part + ((size_t)kp * P.R + r) * P.N + col, v0, v1);
          } else {
            const float s8 = sum8(resid_pair(P, r, col, v0, v1));
            if ((p & 7) == 0) P.ss_out[(size_t)r * (P.N >> 4) + (col >> 4)] = s8;
          }
        } else if constexpr (EPI == EPI_SWIGLU) {
          swiglu_pair(P, r, col, v0, v1);
        } else {
          unsigned long long k0, k1;
          lm_pair_keys(P, sm, r, col, v0, v1, qpos[it], k0, k1);
          const unsigned long long k = k0 > k1 ? k0 : k1;
          kmax[it] = k > kmax[it] ? k : kmax[it];
        }
      }
    }
    __syncthreads();  // sAcc is rewritten by the next block
  };
  for (; blk < nblk; blk += GW) pass(b0, s0, blk, blk + GW);
  if constexpr (EPI == EPI_LM) {
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      unsigned long long k = kmax[it];
#pragma unroll
      for (int o = 4; o >= 1; o >>= 1) {
        const unsigned long long t = __shfl_xor(k, o);
        k = t > k ? t : k;
      }
      const int p = tid + it * NT;
      if (p < P.R * 8 * CT && (p & 7) == 0) atomicMax(&P.argkey[p / (8 * CT)], k);
    }
    lm_finish(P, (int)gridDim.x, (float*)sAcc);
  }
  if constexpr (EPI == EPI_RESID) {
    if (parts == 1) return;
    // The parts of this workgroup's blocks are stored.  One arrival per block,
    // all in flight at once; the blocks this workgroup completed (its part
    // arrived last) are then gathered together: each pair's parts added in
    // part order, then the epilogue.  (Block by block, the arrival and the
    // gather cost two memory round trips per block in series.)
    wait_mem();
    __syncthreads();
    constexpr int CH = 64;  // blocks per round
    const int nmine = wg < nblk ? (nblk - 1 - wg) / GW + 1 : 0;
    for (int i0 = 0; i0 < nmine; i0 += CH) {
      if (tid == 0) sLast = 0;
      __syncthreads();
      for (int i = tid; i < CH && i0 + i < nmine; i += NT) {
        const int b = wg + (i0 + i) * GW;
        const unsigned old = atomicAdd(&P.cnt[b], 1u);
        if (old == (unsigned)(parts - 1)) {
          P.cnt[b] = 0u;  // every part has arrived: ready for the next launch
          sDone[atomicAdd(&sLast, 1)] = b;
        }
      }
      __syncthreads();
      const int nd = sLast, npairs = P.R * 8 * CT;
      // q = block index * npairs + pair: every aligned 8 of q are 16 columns
      // of one row of one block (the shuffle group of the epilogue)
      for (int q = tid; q < nd * npairs; q += NT) {
#pragma clang fp contract(off)
        const int bi = q / npairs, p = q - bi * npairs, b = sDone[bi];
        const int r = p / (8 * CT), rem = p - r * (8 * CT), ct = rem >> 3, pp = rem & 7;
        const int col = (b * CT + ct) * 16 + 2 * pp;
        float2 t[kMmqrMaxParts];
#pragma unroll
        for (int s = 0; s < kMmqrMaxParts; ++s)
          if (s < parts) t[s] = ld_dev2(P.part + ((size_t)s * P.R + r) * P.N + col);
        float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
        for (int s = 0; s < kMmqrMaxParts; ++s)
          if (s < parts) {
            v0 += t[s].x;
            v1 += t[s].y;
          }
        const float s8 = sum8(resid_pair(P, r, col, v0, v1));
        if ((p & 7) == 0) P.ss_out[(size_t)r * (P.N >> 4) + (col >> 4)] = s8;
      }
      __syncthreads();  // sLast and sDone are rewritten by the next round
    }
  }
}

// -------------------------------------------------------------- attention
//
// Grid (split, kv head, sequence x group of tpw query tiles).  A split is
// 256 keys at absolute positions [256*split, 256*split + 256), one 64-key
// chunk (four 16-token blocks) per wave; a query tile is 16 query columns
// (span row, head of the GQA group) of one sequence and kv head.  With
// tpw = 1 the tiles of a long span run side by side (few workgroups: batch
// 1); with more, a workgroup takes its tiles one after another on the K and
// V it loaded once (many workgroups: batched steps).  Scores are computed transposed, S^T = K Q^T, so the
// probabilities come out of the MFMA already in the B-operand layout of
// O^T = V^T P^T and never leave registers; V blocks are stored d-major
// ([hd][16 tokens]) so the V^T operand is read straight from memory.  The
// prologue issues every load unconditionally from clamped addresses (block
// ids, then K, V and the queries) and zeroes what lies past the context
// afterwards, so a workgroup waits for two memory latencies, not one per
// block.  Each wave's chunk softmax is combined across the four waves in LDS
// in wave order and each split's (max, sum, o) goes to memory; the splits of
// a column are merged by combine_tile, run by the tile's last split to
// finish when every context of the step is short, else by k_attn_combine.
// Row i attends keys [0, p+i]; a chunk or split lying wholly past a row's
// position contributes exactly nothing.

template <int HD, bool COH, int MS>
__device__ void combine_tile(const AttnParams& P, int b, int kvh, int qt, int p, float* sML);
constexpr int kMaxCombineSplits = 256;  // host-checked: max_ctx <= 65536

// Two waves per SIMD also with two tiles per pass (a few registers spill).
template <int HD, int TP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn(AttnParams P) {
  static_assert(TP == 1 || TP == 2, "one or two query tiles per pass");
  constexpr int KST = (HD + 31) / 32;  // 32-wide steps over the head dim (zero padded)
  constexpr int DT = HD / 16;          // 16-row tiles of O^T
  constexpr int FS = attn_fuse_splits(HD);
  static_assert(16 * FS * 2 <= TP * 4 * 16 * (HD + 1), "the fused merge's split table fits sO");
  const int kvh = blockIdx.y;
  const int n_tg = (P.n_qt + P.tpw - 1) / P.tpw;  // groups of tpw query tiles
  const int b = blockIdx.z / n_tg, tg = blockIdx.z - b * n_tg;
  const int qt0 = tg * P.tpw, qt1 = min(P.n_qt, qt0 + P.tpw);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int DQ = P.n_q * HD;
  const int S = P.S, G = P.n_q / P.n_kv, QC = S * G;
  // The context length and this wave's four block ids load together (ids
  // clamped to the table row; blocks past the context take the sequence's
  // block 0 and are zeroed below), then K, V and the queries.
  int blk[4];
  int p, total, n_act, split, kb0, s_lo;
  if (P.win) {
    // Sliding window: the ring's block ids follow from the positions, so only
    // the cache length and the sequence id are loaded; the grid starts at the
    // first split the window of row 0 touches.
    p = P.rowinfo[2 * b * S];
    const int seq = P.seq_ids[b];
    total = p + S;
    s_lo = max(0, p - P.win + 1) >> 8;
    split = blockIdx.x + s_lo;
    n_act = ((total - 1) >> 8) - s_lo + 1;
    if ((int)blockIdx.x >= n_act) return;
    kb0 = split * 16 + wave * 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) blk[t] = seq * P.ring_nb + (kb0 + t) % P.ring_nb;
  } else {
    split = blockIdx.x;
    s_lo = 0;
    const int32_t* btrow = P.slotbt + (size_t)b * P.bt_stride;
    kb0 = split * 16 + wave * 4;
    int bv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bv[t] = btrow[kb0 + t < P.bt_stride ? kb0 + t : 0];
    const int bz = btrow[0];
    // every id is loaded before anything branches on the context length
    asm volatile("" ::"v"(bv[0]), "v"(bv[1]), "v"(bv[2]), "v"(bv[3]), "v"(bz));
    p = P.rowinfo[2 * b * S];
    total = p + S;
    n_act = (total + 255) >> 8;
    if (split >= n_act) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) blk[t] = (kb0 + t) * 16 < total ? bv[t] : bz;
  }

  __shared__ float sO[TP][4][16][HD + 1];
  __shared__ float sM[TP][4][16], sL[TP][4][16], sF[TP][4][16];

  // the queries of tile t: 8 fp16 per step and lane (column t*16 + c16)
  auto load_q = [&](u32x4 (&qd)[KST], int t) {
    const int cl = t * 16 + c16, cc = cl < QC ? cl : 0;
    const _Float16* qrow = P.q + (size_t)(b * S + cc / G) * DQ + (kvh * G + cc % G) * HD;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const int d = ks * 32 + g4 * 8, dc = d < HD ? d : 0;
      qd[ks] = *(const u32x4*)(qrow + dc);
    }
  };
  int qt = qt0;
  u32x4 qa[TP][KST];
#pragma unroll
  for (int u = 0; u < TP; ++u) load_q(qa[u], qt0 + u < qt1 ? qt0 + u : qt0);
  f16x8 kf[4][KST];
  f16x4 vf[4][DT];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const _Float16* kbase = P.kpool + ((size_t)blk[t] * P.n_kv + kvh) * 16 * HD;
    const _Float16* vbase = P.vpool + ((size_t)blk[t] * P.n_kv + kvh) * HD * 16;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const int d = ks * 32 + g4 * 8, dc = d < HD ? d : 0;
      kf[t][ks] = *(const f16x8*)(kbase + c16 * HD + dc);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[t][dt] = *(const f16x4*)(vbase + (dt * 16 + c16) * 16 + g4 * 4);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bool ok = (kb0 + t) * 16 < total;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const bool dok = ks * 32 + g4 * 8 < HD;
      kf[t][ks] = (ok && dok) ? kf[t][ks] : (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[t][dt] = ok ? vf[t][dt] : (f16x4){0, 0, 0, 0};
  }
  // The group's query tiles, TP at a time on the same K and V (the tiles of
  // a pass interleave their independent MFMA and softmax chains); each pass's
  // queries load while the previous pass computes.  Every column's arithmetic
  // is the same whatever TP and the pass it falls in.
  for (;;) {
  f16x8 qf[TP][KST];
  bool qok[TP];
  int pos_q[TP];
#pragma unroll
  for (int u = 0; u < TP; ++u) {
    const int cl = (qt + u) * 16 + c16;
    qok[u] = qt + u < qt1 && cl < QC;
    pos_q[u] = p + (qok[u] ? cl : 0) / G;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const bool use = qok[u] && ks * 32 + g4 * 8 < HD;
      qf[u][ks] = __builtin_bit_cast(f16x8, use ? qa[u][ks] : (u32x4){0u, 0u, 0u, 0u});
    }
  }
  if (qt + TP < qt1) {
#pragma unroll
    for (int u = 0; u < TP; ++u) load_q(qa[u], qt + TP + u < qt1 ? qt + TP + u : qt + TP);
  }

  float sc[TP][4][4];
  float mx[TP];
#pragma unroll
  for (int u = 0; u < TP; ++u) mx[u] = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc[TP];
#pragma unroll
    for (int u = 0; u < TP; ++u) acc[u] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KST; ++ks)
#pragma unroll
      for (int u = 0; u < TP; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[t][ks], qf[u][ks], acc[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < TP; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = (kb0 + t) * 16 + g4 * 4 + i;
        const bool vis = qok[u] && key <= pos_q[u] && (P.win == 0 || key > pos_q[u] - P.win);
        sc[u][t][i] = vis ? acc[u][i] * P.scale : -INFINITY;
        mx[u] = fmaxf(mx[u], sc[u][t][i]);
      }
  }
  float l[TP];
  f16x8 pf[TP][2];
#pragma unroll
  for (int u = 0; u < TP; ++u) {
    mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], 16));
    mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], 32));
    l[u] = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = (mx[u] == -INFINITY) ? 0.0f : expf(sc[u][t][i] - mx[u]);
        l[u] += e;
        pf[u][t >> 1][(t & 1) * 4 + i] = (_Float16)e;
      }
    l[u] += __shfl_xor(l[u], 16);
    l[u] += __shfl_xor(l[u], 32);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x4 acc[TP];
#pragma unroll
    for (int u = 0; u < TP; ++u) acc[u] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f16x4 v0 = vf[2 * s2][dt], v1 = vf[2 * s2 + 1][dt];
      const f16x8 a = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int u = 0; u < TP; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[u][s2], acc[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < TP; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) sO[u][wave][c16][dt * 16 + g4 * 4 + i] = acc[u][i];
  }
  if (g4 == 0) {
#pragma unroll
    for (int u = 0; u < TP; ++u) {
      sM[u][wave][c16] = mx[u];
      sL[u][wave][c16] = l[u];
    }
  }
  __syncthreads();
  // Combine the four chunks of this split, in wave order: the weight of
  // each (wave, column) once, then the values.
  if (tid < 16 * TP) {
    const int u = tid >> 4, c = tid & 15;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sM[u][w][c]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (M == -INFINITY) ? 0.0f : expf(sM[u][w][c] - M);
      sF[u][w][c] = f;
      L = __builtin_fmaf(sL[u][w][c], f, L);
    }
    const int qcol = (qt + u) * 16 + c;
    if (qt + u < qt1 && qcol < QC) {
      float* dst = P.part + (((size_t)kvh * P.max_splits + split) * (P.n_seq * QC) + b * QC + qcol) * (HD + 2);
      // device-coherent stores only where another workgroup of this kernel
      // reads them (the fused merge); the merge kernel reads after the launch
      if (P.fuse) {
        st_dev(dst, M);
        st_dev(dst + 1, L);
      } else {
        *(float2*)dst = make_float2(M, L);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < TP * 16 * (HD / 2); e += 256) {
    const int u = e / (16 * (HD / 2)), eu = e - u * (16 * (HD / 2));
    const int c = eu / (HD / 2), d = 2 * (eu % (HD / 2));
    const int qcol = (qt + u) * 16 + c;
    if (qt + u >= qt1 || qcol >= QC) continue;
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = sF[u][w][c];
      o0 = __builtin_fmaf(sO[u][w][c][d], f, o0);
      o1 = __builtin_fmaf(sO[u][w][c][d + 1], f, o1);
    }
    float* dst = P.part + (((size_t)kvh * P.max_splits + split) * (P.n_seq * QC) + b * QC + qcol) * (HD + 2);
    if (P.fuse) st_dev2(dst + 2 + d, o0, o1);
    else *(float2*)(dst + 2 + d) = make_float2(o0, o1);
  }
  qt += TP;
  if (qt >= qt1) break;
  __syncthreads();  // sO, sM, sL and sF are rewritten by the next pass
  }
  if (!P.fuse) return;
  // Short contexts: the last split of this (sequence, kv head, tile group)
  // to finish merges the group's columns, as k_attn_combine would.
  __shared__ int sLast;
  wait_mem();
  __syncthreads();
  unsigned* cnt = P.cnt + ((size_t)b * P.n_kv + kvh) * n_tg + tg;
  if (tid == 0) {
    const unsigned old = atomicAdd(cnt, 1u);
    sLast = old == (unsigned)(n_act - 1);
  }
  __syncthreads();
  if (!sLast) return;
  if (tid == 0) *cnt = 0u;  // ready for the next launch
  for (int t = qt0; t < qt1; ++t) combine_tile<HD, true, FS>(P, b, kvh, t, p, &sO[0][0][0][0]);
}

template <bool COH>
__device__ __forceinline__ float2 ld_part2(const float* p) {
  if constexpr (COH) return ld_dev2(p);
  else return *(const float2*)p;
}

// Split merge of the 16 query columns of tile qt (sequence b, kv head kvh)
// by 256 threads: column c = tid / 16 belongs to 16 threads of one wave,
// which hold its splits j, j + 16, ... for the maxima and its output pairs
// j, j + 16, ... for the sums.  Per column: M = the largest split maximum;
// f_s = exp(m_s - M); L = the sum of l_s f_s in split order; o = the sum
// of o_s (f_s (1/L)) in split order.  Every order depends only on the
// column's own row position, never on the other rows.  p is the sequence's
// cache length; sML holds 16 x MS (f, l) pairs of LDS (MS >= the column's
// splits).  The maxima, then the first 16 splits' outputs, are loaded
// before anything waits.  COH: the partials were written by other
// workgroups of the same kernel (device-coherent loads).
template <int HD, bool COH, int MS>
__device__ void combine_tile(const AttnParams& P, int b, int kvh, int qt, int p, float* sML) {
#pragma clang fp contract(off)
  static_assert(MS % 16 == 0, "whole rounds of 16 splits");
  constexpr int PP = HD >= 32 ? HD / 32 : 1;  // output pairs per thread
  constexpr int CH = 16;                      // splits of output loads in flight
  const int tid = threadIdx.x, c = tid >> 4, j = tid & 15;
  const int G = P.n_q / P.n_kv, QC = P.S * G;
  const int qcol = qt * 16 + c;
  const bool cok = qcol < QC;
  const int qc = cok ? qcol : 0;
  const int iq = qc / G, head = kvh * G + qc % G;
  // the column's splits: from the first its window touches (0 unless the
  // layer has a sliding window) to the one holding its own position
  const int sp0 = P.win ? max(0, p + iq - P.win + 1) >> 8 : 0;
  int nsp = cok ? ((p + iq) >> 8) + 1 - sp0 : 0;
  nsp = nsp < MS ? nsp : MS;
  const size_t stride = (size_t)(P.n_seq * QC) * (HD + 2);
  const float* base = P.part + ((size_t)kvh * P.max_splits * (P.n_seq * QC) + b * QC + qc) * (HD + 2) +
                      (size_t)sp0 * stride;
  float* ml = sML + (size_t)c * MS * 2;

  float2 mlv[MS / 16];
#pragma unroll
  for (int it = 0; it < MS / 16; ++it) {
    const int sp = j + 16 * it;
    mlv[it] = ld_part2<COH>(base + (size_t)(sp < nsp ? sp : 0) * stride);
  }
  float2 v[PP][CH];
#define SPECV_COMBINE_LOADS(s0)                                                  \
  _Pragma("unroll") for (int i = 0; i < PP; ++i) {                               \
    const int dp = j + 16 * i, dpc = dp < HD / 2 ? dp : 0;                       \
    _Pragma("unroll") for (int k = 0; k < CH; ++k) {                             \
      const int sp = (s0) + k < nsp ? (s0) + k : 0;                              \
      v[i][k] = ld_part2<COH>(base + (size_t)sp * stride + 2 + 2 * dpc);         \
    }                                                                            \
  }
  SPECV_COMBINE_LOADS(0)
  float M = -INFINITY;
#pragma unroll
  for (int it = 0; it < MS / 16; ++it) {
    const int sp = j + 16 * it;
    if (sp < nsp) {
      ml[2 * sp] = mlv[it].x;
      ml[2 * sp + 1] = mlv[it].y;
      M = fmaxf(M, mlv[it].x);
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the column's maxima and sums are in LDS
  for (int sp = j; sp < nsp; sp += 16) ml[2 * sp] = expf(ml[2 * sp] - M);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);
  float L = 0.0f;
  for (int sp = 0; sp < nsp; ++sp) L += ml[2 * sp + 1] * ml[2 * sp];
  const float inv = 1.0f / L;
  float o0[PP], o1[PP];
#pragma unroll
  for (int i = 0; i < PP; ++i) o0[i] = o1[i] = 0.0f;
  for (int s0 = 0; s0 < nsp; s0 += CH) {
    if (s0 > 0) { SPECV_COMBINE_LOADS(s0) }
#pragma unroll
    for (int k = 0; k < CH; ++k)
      if (s0 + k < nsp) {
        const float w = ml[2 * (s0 + k)] * inv;
#pragma unroll
        for (int i = 0; i < PP; ++i) {
          o0[i] += v[i][k].x * w;
          o1[i] += v[i][k].y * w;
        }
      }
  }
#undef SPECV_COMBINE_LOADS
  const int DQ = P.n_q * HD;
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const int dp = j + 16 * i;
    if (cok && dp < HD / 2) {
      const size_t oi = (size_t)(b * P.S + iq) * DQ + head * HD + 2 * dp;
      *(float2*)(P.out + oi) = make_float2(o0[i], o1[i]);
      if (P.out16) {
        const _Float16 h0 = (_Float16)o0[i], h1 = (_Float16)o1[i];
        *(uint32_t*)(P.out16 + oi) =
            (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      }
      if (P.af_out) prep_store2(P.af_out, (P.n_seq * P.S + 15) >> 4, b * P.S + iq, head * HD + 2 * dp, o0[i], o1[i]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Split merge kernel for long contexts: grid (query tile, kv head, sequence).
template <int HD>
__global__ __launch_bounds__(256) void k_attn_combine(AttnParams P) {
  __shared__ float sML[16 * kMaxCombineSplits * 2];
  const int b = blockIdx.z;
  combine_tile<HD, false, kMaxCombineSplits>(P, b, blockIdx.y, blockIdx.x, P.rowinfo[2 * b * P.S], sML);
}

// ------------------------------------------------------- recurrent layer
//
// A delta-rule layer (TensorSharp page, recurrent-trunk section): per kv head
// a state S [hd (v)][hd (k)] that every row updates, S <- S + beta (v - S k)
// k^T with the row's unit key k, and every query head of the group reads,
// o = S q with the unit query q.  One workgroup per (kv head, sequence) holds
// S in registers (thread t: row t / TPR, columns (t % TPR) * E .. + E) and runs
// the span's rows in order; after each row it stores S as that row's
// snapshot, so the accept stage can commit the state after any row by index
// (the page: keep one snapshot per row, commit it on the device, and the
// pre-verify state is simply the one not overwritten).  Every sum runs in a
// fixed order per row, whatever the span, so the rows gate holds.
template <int HD>
__global__ __launch_bounds__(256) void k_recur(RecParams P) {
  constexpr int E = HD * HD / 256, TPR = HD / E;  // state elements per thread, threads per state row
  constexpr int MAXG = 8;                        // query heads per kv head held in the LDS
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dv = tid / TPR, dk0 = (tid % TPR) * E;
  const int G = P.n_q / P.n_kv, DQ = P.n_q * HD, DK = P.n_kv * HD;
  const int seq = P.seq_ids[b];
  __shared__ float sX[(2 + MAXG) * HD];  // k, q_0..q_(G-1), then v
  __shared__ float sN[1 + MAXG];
  float* sV = sX + (1 + MAXG) * HD;
  const int old = P.slot[seq];
  const int set = old < 0 ? 0 : 1 - (old >> 4);
  float S[E];
  if (old < 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) S[e] = 0.0f;
  } else {
    const float* src = P.snap + ((((size_t)seq * 2 + (old >> 4)) * 16 + (old & 15)) * P.n_kv + g) * HD * HD +
                       (size_t)dv * HD + dk0;
#pragma unroll
    for (int e = 0; e < E; ++e) S[e] = src[e];
  }
  for (int i = 0; i < P.S; ++i) {
    const int r = b * P.S + i;
    // the row's key, queries and value
    for (int e = tid; e < (2 + G) * HD; e += 256) {
      const int v = e / HD, d = e % HD;
      float x;
      if (v == 0) x = P.kv[(size_t)r * 2 * DK + g * HD + d];
      else if (v <= G) x = P.q[(size_t)r * DQ + (g * G + v - 1) * HD + d];
      else x = P.kv[(size_t)r * 2 * DK + DK + g * HD + d];
      if (v <= G) sX[v * HD + d] = x;
      else sV[d] = x;
    }
    __syncthreads();
    // lengths of the key and the queries: one wave each, lanes over d, xor tree
    for (int v = wave; v <= G; v += 4) {
      float a = 0.0f;
      for (int d = lane; d < HD; d += 64) a += sX[v * HD + d] * sX[v * HD + d];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
      if (lane == 0) sN[v] = sqrtf(a);
    }
    __syncthreads();
    for (int e = tid; e < (1 + G) * HD; e += 256) sX[e] = sX[e] / sN[e / HD];
    __syncthreads();
    // u = S k (this thread's part, then the TPR threads of the row), the write
    float u = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) u += S[e] * sX[dk0 + e];
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) u += __shfl_xor(u, o);
    const float cw = P.beta * (sV[dv] - u);
#pragma unroll
    for (int e = 0; e < E; ++e) S[e] = S[e] + cw * sX[dk0 + e];
    float* dst = P.snap + ((((size_t)seq * 2 + set) * 16 + i) * P.n_kv + g) * HD * HD + (size_t)dv * HD + dk0;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = S[e];
    // the reads of the group's queries
    for (int h = 0; h < G; ++h) {
      float o = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) o += S[e] * sX[(1 + h) * HD + dk0 + e];
#pragma unroll
      for (int x = TPR / 2; x >= 1; x >>= 1) o += __shfl_xor(o, x);
      if (tid % TPR == 0) {
        const int col = (g * G + h) * HD + dv;
        P.out[(size_t)r * DQ + col] = o;
        if (P.af_out) prep_store1(P.af_out, (P.n_seq * P.S + 15) >> 4, r, col, o);
      }
    }
    __syncthreads();  // the LDS is refilled for the next row
  }
}

hipError_t launch_recur(const RecParams& p, int hd, hipStream_t st) {
  if (!p.q || !p.kv || !p.snap || !p.slot || !p.seq_ids || !p.out || p.n_kv < 1 || p.n_q % p.n_kv ||
      p.n_q / p.n_kv > 8 || p.S < 1 || p.S > 16 || p.n_seq < 1)
    return hipErrorInvalidValue;
  const dim3 grid(p.n_kv, p.n_seq);
  switch (hd) {
    case 128: hipLaunchKernelGGL(k_recur<128>, grid, dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL(k_recur<64>, grid, dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL(k_recur<32>, grid, dim3(256), 0, st, p); break;
    case 16: hipLaunchKernelGGL(k_recur<16>, grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------- streaming read
//
// The measured read peak: every workgroup streams its share of a buffer with
// 16-byte non-temporal loads, eight in flight per thread, and folds them into
// one word per thread (written only if it is a sentinel no data produces, so
// the loads cannot be dropped).  Grid = a multiple of the CU count.
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, size_t n16,
                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 255] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t st) {
  if (!src || !sink || bytes < 16 || bytes % 16 || ((uintptr_t)src & 15) || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, st, (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

// -------------------------------------------------------------- launchers

template <int EPI>
static hipError_t launch_gemm_epi(const GemmParams& p, int nk, int fmt, hipStream_t st) {
  const int bw = 64 * gemm_tiles_per_wave(fmt);
  const int NB = (p.N + bw - 1) / bw;
  const int grid = ((NB + 7) / 8) * 8 * p.nslices;
  if (fmt == FMT_INT4) {
    if (!p.scales) return hipErrorInvalidValue;
    switch (nk) {
      case 16: hipLaunchKernelGGL((k_gemm<16, EPI, FMT_INT4>), dim3(grid), dim3(256), 0, st, p); break;
      case 8: hipLaunchKernelGGL((k_gemm<8, EPI, FMT_INT4>), dim3(grid), dim3(256), 0, st, p); break;
      case 4: hipLaunchKernelGGL((k_gemm<4, EPI, FMT_INT4>), dim3(grid), dim3(256), 0, st, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (fmt != FMT_BF16) return hipErrorInvalidValue;
  if (p.Af) return hipErrorInvalidValue;  // prepared A is the many-row GEMM's (launch_gemm_big)
  switch (nk) {
    case 19: hipLaunchKernelGGL((k_gemm<19, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    case 16: hipLaunchKernelGGL((k_gemm<16, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    case 10: hipLaunchKernelGGL((k_gemm<10, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    case 8: hipLaunchKernelGGL((k_gemm<8, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    case 5: hipLaunchKernelGGL((k_gemm<5, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    case 4: hipLaunchKernelGGL((k_gemm<4, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((k_gemm<2, EPI, FMT_BF16>), dim3(grid), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Activation rows once in the 16x16x32 MFMA A-operand order, for the
// many-row GEMM: entry (ks * nch + ch) * 64 + l (16 bytes) holds, for lane l,
// row 16 ch + l % 16 and inputs 32 ks + 8 (l / 16) .. +8 as fp16; rows past R
// are zero.  The RMSNorm is the one every GEMM applies (rstd16, then
// (x * rstd) * gain), with the same fp16 rounding.  Grid (ceil(K/512),
// ceil(R/16)): 16 steps of one 16-row chunk per workgroup.
constexpr int kPrepSs = 32;  // RMSNorm partial sums per lane in k_prep: hidden <= 16 * 16 * 32

__global__ __launch_bounds__(256) void k_prep(GemmParams P, u32x4* af) {
  const int ch = blockIdx.y, nch = gridDim.y, ks0 = blockIdx.x * 16, KS = P.K / 32;
  const int tid = threadIdx.x;
  const bool norm = P.ss != nullptr;
  __shared__ float sR[16];
  // Every load first, from clamped addresses (zeroed after): the chunk's
  // RMSNorm statistics (16 lanes per row, as rstd16), its rows, the gains.
  const int sr = ch * 16 + (tid >> 4), sj = tid & 15, src = sr < P.R ? sr : 0;
  // without the RMSNorm, the statistics and gain loads read A (valid memory, values unused)
  const float* ssp = norm ? P.ss + (size_t)src * P.ss_n : P.A;
  const float* gp = norm ? P.gain : P.A;
  const int ssn = norm ? P.ss_n : 1;
  float sv[kPrepSs];
#pragma unroll
  for (int i = 0; i < kPrepSs; ++i) {
    const int q = sj + 16 * i;
    sv[i] = ssp[q < ssn ? q : 0];
  }
  f32x4 a[4][2], gg[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + i * 256, l = u & 63, ks = ks0 + (u >> 6);
    const int r = ch * 16 + (l & 15), g = l >> 4, kc = ks < KS ? ks : 0;
    const f32x4* src_a = (const f32x4*)(P.A + (size_t)(r < P.R ? r : 0) * P.lda + kc * 32 + g * 8);
    a[i][0] = src_a[0];
    a[i][1] = src_a[1];
    const f32x4* src_g = (const f32x4*)(gp + (norm ? kc * 32 + g * 8 : 0));
    gg[i][0] = src_g[0];
    gg[i][1] = src_g[1];
  }
  asm volatile("" ::: "memory");  // every load above is issued before any is used
  if (norm) {
    float acc = 0.0f;  // rstd16's order: partials j, j + 16, ... (zeros past the row), then the xor tree
#pragma unroll
    for (int i = 0; i < kPrepSs; ++i) {
      const unsigned keep = (sr < P.R && sj + 16 * i < P.ss_n) ? ~0u : 0u;  // a mask, not a branch
      acc += __uint_as_float(__float_as_uint(sv[i]) & keep);
    }
    const float rs = rstd_finish(acc, P.inv_dim, P.eps);
    if (sj == 0) sR[tid >> 4] = sr < P.R ? rs : 0.0f;
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + i * 256, l = u & 63, ks = ks0 + (u >> 6);
    const int row = l & 15, r = ch * 16 + row;
    if (ks < KS) {
      float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      if (r < P.R) {
        v[0] = a[i][0].x; v[1] = a[i][0].y; v[2] = a[i][0].z; v[3] = a[i][0].w;
        v[4] = a[i][1].x; v[5] = a[i][1].y; v[6] = a[i][1].z; v[7] = a[i][1].w;
      }
      if (norm) {
        const float rs = sR[row];
        const float gv[8] = {gg[i][0].x, gg[i][0].y, gg[i][0].z, gg[i][0].w,
                             gg[i][1].x, gg[i][1].y, gg[i][1].z, gg[i][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (v[e] * rs) * gv[e];
      }
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[e];
      af[((size_t)ks * nch + ch) * 64 + l] = __builtin_bit_cast(u32x4, h);
    }
  }
}

hipError_t launch_prep_a(const GemmParams& p, void* af, hipStream_t st) {
  if (!af || !p.A || p.R < 1 || p.K % 32 || p.lda % 4 || (p.ss && (!p.gain || p.ss_n > 16 * kPrepSs)))
    return hipErrorInvalidValue;
  const dim3 grid((p.K / 32 + 15) / 16, (p.R + 15) / 16);
  hipLaunchKernelGGL(k_prep, grid, dim3(256), 0, st, p, (u32x4*)af);
  return hipGetLastError();
}

// The many-row GEMM: ns slices of K (ns > 1: partials, then k_gather),
// ct tiles per wave, pd steps in flight.
template <int EPI, int CT, int PD>
static hipError_t go_big(const GemmParams& p, hipStream_t st) {
  const int NB = (p.N + 64 * CT - 1) / (64 * CT);
  const int ksl = p.K / 32 / p.nslices;
  if (ksl % PD) return hipErrorInvalidValue;
  const int grid = ((NB + 7) / 8) * 8 * p.nslices;
  hipLaunchKernelGGL((k_gemm_big<EPI, CT, PD>), dim3(grid), dim3(256), 0, st, p, ksl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nslices == 1) return e;
  if constexpr (EPI != EPI_LM) {
    const long long pairs = (long long)p.R * (((p.N >> 1) + 7) & ~7);
    hipLaunchKernelGGL((k_gather<EPI>), dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

template <int EPI>
static hipError_t launch_big_epi(const GemmParams& p, int ct, hipStream_t st) {
  if (ct == 2) return go_big<EPI, 2, SPECV_BIG_PD2>(p, st);
  return go_big<EPI, 1, SPECV_BIG_PD1>(p, st);
}

hipError_t launch_gemm_big(const GemmParams& p, int ns, int ct, int epi, hipStream_t st) {
  if (!p.Af || !p.W || p.R <= 16 || p.R > kMaxRows || p.K % 32 || ns < 1 || (p.K / 32) % ns || (ct != 1 && ct != 2))
    return hipErrorInvalidValue;
  if (ns > 1 && (epi == EPI_LM || p.N % 16 || !p.part)) return hipErrorInvalidValue;
  if (epi == EPI_QKV && !p.rowinfo) return hipErrorInvalidValue;
  if (epi == EPI_LM && (!p.kd || !p.step || !p.rowinfo || !p.seq_ids || !p.argkey || !p.lm_cnt)) return hipErrorInvalidValue;
  GemmParams q = p;
  q.nslices = ns;
  switch (epi) {
    case EPI_QKV: return launch_big_epi<EPI_QKV>(q, ct, st);
    case EPI_RESID: return launch_big_epi<EPI_RESID>(q, ct, st);
    case EPI_SWIGLU: return launch_big_epi<EPI_SWIGLU>(q, ct, st);
    case EPI_LM: return launch_big_epi<EPI_LM>(q, ct, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmParams& p, int nk, int epi, int fmt, hipStream_t st) {
  if (epi == EPI_QKV && !p.rowinfo) return hipErrorInvalidValue;
  if (epi == EPI_LM && (!p.kd || !p.step || !p.rowinfo || !p.seq_ids)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV: return launch_gemm_epi<EPI_QKV>(p, nk, fmt, st);
    case EPI_RESID: return launch_gemm_epi<EPI_RESID>(p, nk, fmt, st);
    case EPI_SWIGLU: return launch_gemm_epi<EPI_SWIGLU>(p, nk, fmt, st);
    case EPI_LM: return launch_gemm_epi<EPI_LM>(p, nk, fmt, st);
  }
  return hipErrorInvalidValue;
}

// The compiled one-pass configurations (waves = K parts, steps per part,
// tiles per workgroup) of each epilogue class.
// nbuf 1 or 2: the walking k_mm with ct-tile blocks; nbuf 0: k_mm1, one tile
// per workgroup, loaded in ct phases.
// (nw, spw, ct, nbuf, gp): gp parts per group of the final sum.
#define SPECV_MM_H(X) X(16, 5, 1, 1, 16) X(1, 2, 1, 1, 1) X(2, 1, 1, 1, 2)
#define SPECV_MM_R(X) X(8, 16, 2, 0, 1) X(16, 8, 1, 0, 1) X(16, 19, 4, 0, 1) X(1, 2, 1, 1, 1) X(2, 1, 1, 1, 2) \
  X(1, 4, 1, 1, 1) X(2, 2, 1, 1, 2) X(4, 1, 1, 1, 4)

bool mm_supported(int epi, int nw, int spw, int ct, int nbuf, int gp) {
#define SPECV_MM_HAS(a, b, c, d, e) if (nw == a && spw == b && ct == c && nbuf == d && gp == e) return true;
  if (epi == EPI_QKV || epi == EPI_SWIGLU || epi == EPI_LM) {
    SPECV_MM_H(SPECV_MM_HAS)
  } else if (epi == EPI_RESID) {
    SPECV_MM_R(SPECV_MM_HAS)
  }
#undef SPECV_MM_HAS
  return false;
}

// int4 one-pass (k_mmq) configurations: (waves, groups per wave, 16-column
// tiles per pass).  K = 5120 takes eight waves of five groups, the K parts of
// the register-activation kernel that serves nine to sixteen rows, so the
// two agree bit for bit (ten waves of four ran 1-6 % faster at one row: LM
// head 93 vs 99 us).  Two tiles per pass share each read of the A slice from
// LDS where the LDS holds the second partial tile (K = 5120: 80 KiB of A for
// eight fp16 rows + 16 KiB of partials; K = 8192 has 128 KiB of A and no room
// for it); they are taken when
// every workgroup walks at least four such blocks (gate/up 46.9 -> 42.6 us,
// LM head 129 -> 110 us at the 32B shape), since with fewer the blocks split
// unevenly over the workgroups (QKV's 640 tiles: 16.4 -> 18.0 us).
#ifndef SPECV_MMQ_CT
#define SPECV_MMQ_CT 2
#endif
// (waves, groups per wave, tiles per pass, residual epilogue only): sixteen
// waves of four groups serve O (K = 8192) alone, whose staging holds no gains.
#define SPECV_MMQ(X) X(8, 5, 1, 0) X(8, 5, SPECV_MMQ_CT, 0) X(16, 4, 1, 1) X(1, 1, 1, 0)

bool mmq_supported(int K, int nk, int epi) {
  if (nk % 4 || K % (32 * nk)) return false;
  const int gpw = nk / 4, nw = K / (32 * nk);
#define SPECV_MMQ_HAS(a, b, c, ro) \
  if (nw == a && gpw == b && (!(ro) || epi == EPI_RESID)) return true;
  SPECV_MMQ(SPECV_MMQ_HAS)
#undef SPECV_MMQ_HAS
  return false;
}

// One k_mmq configuration's launch; a residual-only configuration is never
// instantiated with another epilogue.
template <int EPI, int NW, int GPW, int CT, bool RO>
hipError_t go_mmq(dim3 grid, const GemmParams& p, hipStream_t st) {
  if constexpr (RO && EPI != EPI_RESID) {
    return hipErrorInvalidValue;
  } else {
    // four staged rows where they suffice (less staging work at one row)
    if constexpr (EPI == EPI_RESID) {
      if (p.A16) {  // the rows already rounded to fp16
        if (p.R <= 4) hipLaunchKernelGGL((k_mmq<EPI, NW, GPW, CT, 4, true>), grid, dim3(NW * 64), 0, st, p);
        else hipLaunchKernelGGL((k_mmq<EPI, NW, GPW, CT, 8, true>), grid, dim3(NW * 64), 0, st, p);
        return hipGetLastError();
      }
    } else {
      if (p.A16) return hipErrorInvalidValue;
    }
    if (p.R <= 4) hipLaunchKernelGGL((k_mmq<EPI, NW, GPW, CT, 4>), grid, dim3(NW * 64), 0, st, p);
    else hipLaunchKernelGGL((k_mmq<EPI, NW, GPW, CT, 8>), grid, dim3(NW * 64), 0, st, p);
    return hipGetLastError();
  }
}

hipError_t launch_mmq(const GemmParams& p, int nk, int epi, int max_grid, hipStream_t st) {
  if (p.R < 1 || p.R > 8 || !p.scales || p.N % 16 || max_grid < 1 || !mmq_supported(p.K, nk, epi))
    return hipErrorInvalidValue;
  if (epi != EPI_RESID && (!p.ss || !p.gain || p.ss_n * 16 != p.K)) return hipErrorInvalidValue;
  if (epi == EPI_QKV && !p.rowinfo) return hipErrorInvalidValue;
  if (epi == EPI_LM && (!p.argkey || !p.lm_cnt || !p.status || !p.result || !p.kd || !p.step || !p.rowinfo || p.R != p.n_seq * p.S))
    return hipErrorInvalidValue;
  const int gpw = nk / 4, nw = p.K / (32 * nk), ntile = p.N / 16;
  const int ct = (nw == 8 && ntile >= 8 * max_grid) ? SPECV_MMQ_CT : 1;
#define SPECV_MMQ_GO(a, b, c, ro)                                                  \
  if (nw == a && gpw == b && ct == (c)) {                                          \
    const int nblk = (ntile + (c) - 1) / (c);                                      \
    const dim3 grid(nblk < max_grid ? nblk : max_grid);                            \
    switch (epi) {                                                                 \
      case EPI_QKV: return go_mmq<EPI_QKV, a, b, c, (ro) != 0>(grid, p, st);       \
      case EPI_RESID: return go_mmq<EPI_RESID, a, b, c, (ro) != 0>(grid, p, st);   \
      case EPI_SWIGLU: return go_mmq<EPI_SWIGLU, a, b, c, (ro) != 0>(grid, p, st); \
      case EPI_LM: return go_mmq<EPI_LM, a, b, c, (ro) != 0>(grid, p, st);         \
      default: return hipErrorInvalidValue;                                        \
    }                                                                              \
  }
  SPECV_MMQ(SPECV_MMQ_GO)
#undef SPECV_MMQ_GO
  return hipErrorInvalidValue;
}

// int4 register-A one-pass (k_mmqr) configurations: (waves, groups of 128
// inputs per wave); a wave holds 4 * GPW steps of activations (8 registers
// each), so GPW <= 5 with eight waves keeps two waves per SIMD.  K is covered
// by K / (128 * NW * GPW) workgroup parts, at most kMmqrMaxParts.
#define SPECV_MMQR(X) X(8, 5) X(8, 4) X(4, 1) X(2, 1) X(1, 1)

bool mmqr_plan(int K, int* nw, int* gpw, int* parts) {
  if (K <= 0 || K % 128) return false;
  const int groups = K / 128;
#define SPECV_MMQR_PLAN(a, b)                                      \
  if (groups % ((a) * (b)) == 0 && groups / ((a) * (b)) <= kMmqrMaxParts) { \
    *nw = (a);                                                     \
    *gpw = (b);                                                    \
    *parts = groups / ((a) * (b));                                 \
    return true;                                                   \
  }
  SPECV_MMQR(SPECV_MMQR_PLAN)
#undef SPECV_MMQR_PLAN
  return false;
}

#ifndef SPECV_MMQR_CT
#define SPECV_MMQR_CT 1
#endif

hipError_t launch_mmqr(const GemmParams& p0, int epi, int max_grid, hipStream_t st) {
  int nw = 0, gpw = 0, parts = 0;
  if (p0.R < 1 || p0.R > 16 || !p0.scales || p0.N % 16 || max_grid < 1 || !mmqr_plan(p0.K, &nw, &gpw, &parts))
    return hipErrorInvalidValue;
  if (parts > 1 && (epi != EPI_RESID || !p0.part || !p0.cnt)) return hipErrorInvalidValue;
  if (epi != EPI_RESID && (!p0.ss || !p0.gain || p0.ss_n * 16 != p0.K)) return hipErrorInvalidValue;
  if (epi != EPI_RESID && p0.A16) return hipErrorInvalidValue;
  if (epi == EPI_RESID && (!p0.x || !p0.ss_out)) return hipErrorInvalidValue;
  if (epi == EPI_QKV && !p0.rowinfo) return hipErrorInvalidValue;
  if (epi == EPI_LM && (!p0.argkey || !p0.lm_cnt || !p0.status || !p0.result || !p0.kd || !p0.step || !p0.rowinfo ||
                        p0.R != p0.n_seq * p0.S))
    return hipErrorInvalidValue;
  GemmParams p = p0;
  p.nslices = parts;
  const int ct = SPECV_MMQR_CT;
  const int nblk = (p.N / 16 + ct - 1) / ct;
  int gw = max_grid / parts;
  gw = gw < 1 ? 1 : (gw < nblk ? gw : nblk);
  const dim3 grid(gw * parts);
#define SPECV_MMQR_GO(a, b)                                                                                   \
  if (nw == (a) && gpw == (b)) {                                                                              \
    switch (epi) {                                                                                            \
      case EPI_QKV: hipLaunchKernelGGL((k_mmqr<EPI_QKV, a, b, SPECV_MMQR_CT>), grid, dim3(a * 64), 0, st, p); break;     \
      case EPI_RESID:                                                                                         \
        if (p.A16) hipLaunchKernelGGL((k_mmqr<EPI_RESID, a, b, SPECV_MMQR_CT, true>), grid, dim3(a * 64), 0, st, p); \
        else hipLaunchKernelGGL((k_mmqr<EPI_RESID, a, b, SPECV_MMQR_CT>), grid, dim3(a * 64), 0, st, p);    \
        break;                                                                                                \
      case EPI_SWIGLU: hipLaunchKernelGGL((k_mmqr<EPI_SWIGLU, a, b, SPECV_MMQR_CT>), grid, dim3(a * 64), 0, st, p); break; \
      case EPI_LM: hipLaunchKernelGGL((k_mmqr<EPI_LM, a, b, SPECV_MMQR_CT>), grid, dim3(a * 64), 0, st, p); break;       \
      default: return hipErrorInvalidValue;                                                                   \
    }                                                                                                         \
    return hipGetLastError();                                                                                 \
  }
  SPECV_MMQR(SPECV_MMQR_GO)
#undef SPECV_MMQR_GO
  return hipErrorInvalidValue;
}

hipError_t launch_mm1l(const GemmParams& p, int nw, int spw, int rl, hipStream_t st) {
  if (p.R < 1 || p.R > rl || p.K != nw * spw * 32 || p.N % 16) return hipErrorInvalidValue;
  // the smallest staging that holds the rows; A from fp16 rows when given
#define SPECV_MM1L_GO(a, b, c)                                                                         \
  do {                                                                                                 \
    if (p.A16) hipLaunchKernelGGL((k_mm1l<a, b, c, true>), dim3(p.N / 16), dim3(a * 64), 0, st, p);   \
    else hipLaunchKernelGGL((k_mm1l<a, b, c, false>), dim3(p.N / 16), dim3(a * 64), 0, st, p);        \
  } while (0)
  if (nw == 16 && spw == 19 && rl == 8) {
    if (p.R <= 2) SPECV_MM1L_GO(16, 19, 2);
    else if (p.R <= 4) SPECV_MM1L_GO(16, 19, 4);
    else SPECV_MM1L_GO(16, 19, 8);
    return hipGetLastError();
  }
  if (nw == 8 && spw == 16 && rl == 4) {
    if (p.R <= 2) SPECV_MM1L_GO(8, 16, 2);
    else SPECV_MM1L_GO(8, 16, 4);
    return hipGetLastError();
  }
#undef SPECV_MM1L_GO
  return hipErrorInvalidValue;
}

hipError_t launch_mm(const GemmParams& p, int nw, int spw, int ct, int nbuf, int gp, int max_grid, int epi,
                     hipStream_t st) {
  if (p.R < 1 || p.R > 16 || p.K != nw * spw * 32 || max_grid < 1 || p.N % 16) return hipErrorInvalidValue;
  // the RMSNorm prologue reads K/16 partial sums per row (K = hidden)
  if ((epi == EPI_QKV || epi == EPI_SWIGLU || epi == EPI_LM) && (!p.ss || !p.gain || p.ss_n * 16 != p.K))
    return hipErrorInvalidValue;
  if (epi == EPI_QKV && !p.rowinfo) return hipErrorInvalidValue;
  if (epi == EPI_LM && (!p.argkey || !p.lm_cnt || !p.status || !p.result || !p.kd || !p.step || !p.rowinfo || p.R != p.n_seq * p.S))
    return hipErrorInvalidValue;
  const int nblk = (p.N + 16 * ct - 1) / (16 * ct), nblk1 = (p.N + 15) / 16;
  const int grid = nblk < max_grid ? nblk : max_grid;
#define SPECV_MM_GO(E, a, b, c, d, e)                                                    \
  if (nw == a && spw == b && ct == c && nbuf == d && gp == e) {                          \
    if constexpr (d == 0) {                                                              \
      if constexpr (E == EPI_RESID) {                                                    \
        if (p.A16) hipLaunchKernelGGL((k_mm1<E, a, b, c, e, true>), dim3(nblk1), dim3(a * 64), 0, st, p); \
        else hipLaunchKernelGGL((k_mm1<E, a, b, c, e, false>), dim3(nblk1), dim3(a * 64), 0, st, p); \
      } else {                                                                           \
        if (p.A16) return hipErrorInvalidValue;                                          \
        hipLaunchKernelGGL((k_mm1<E, a, b, c, e, false>), dim3(nblk1), dim3(a * 64), 0, st, p); \
      }                                                                                  \
    } else                                                                               \
      hipLaunchKernelGGL((k_mm<E, a, b, c, d, e>), dim3(grid), dim3(a * 64), 0, st, p); \
    return hipGetLastError();                                                            \
  }
#define SPECV_MM_GO_Q(a, b, c, d, e) SPECV_MM_GO(EPI_QKV, a, b, c, d, e)
#define SPECV_MM_GO_S(a, b, c, d, e) SPECV_MM_GO(EPI_SWIGLU, a, b, c, d, e)
#define SPECV_MM_GO_R(a, b, c, d, e) SPECV_MM_GO(EPI_RESID, a, b, c, d, e)
#define SPECV_MM_GO_L(a, b, c, d, e) SPECV_MM_GO(EPI_LM, a, b, c, d, e)
  if (epi == EPI_QKV) {
    SPECV_MM_H(SPECV_MM_GO_Q)
  } else if (epi == EPI_SWIGLU) {
    SPECV_MM_H(SPECV_MM_GO_S)
  } else if (epi == EPI_RESID) {
    SPECV_MM_R(SPECV_MM_GO_R)
  } else if (epi == EPI_LM) {
    SPECV_MM_H(SPECV_MM_GO_L)
  }
#undef SPECV_MM_GO_L
#undef SPECV_MM_GO_Q
#undef SPECV_MM_GO_S
#undef SPECV_MM_GO_R
#undef SPECV_MM_GO
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnParams& p, int hd, hipStream_t st) {
  if (p.max_splits > kMaxCombineSplits || p.n_kv < 1 || p.n_q % p.n_kv) return hipErrorInvalidValue;
  const int n_qt = (p.S * (p.n_q / p.n_kv) + 15) / 16;
  if (p.n_qt != n_qt || p.tpw < 1 || p.tpw > n_qt || p.n_seq < 1 || p.n_seq * n_qt > 65535)
    return hipErrorInvalidValue;
  if (p.win && (p.win < 1 || p.ring_nb < 1 || p.ring_w != 16 * p.ring_nb || !p.seq_ids || p.grid_splits < 1 ||
                p.grid_splits > p.max_splits))
    return hipErrorInvalidValue;
  const dim3 grid(p.win ? p.grid_splits : p.max_splits, p.n_kv, p.n_seq * ((n_qt + p.tpw - 1) / p.tpw));
  // workgroups with several query tiles take them two per pass
  const bool two = p.tpw > 1 && n_qt > 1;
  const dim3 cgrid(n_qt, p.n_kv, p.n_seq);
  switch (hd) {
    case 128:
      if (two) hipLaunchKernelGGL((k_attn<128, 2>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_attn<128, 1>), grid, dim3(256), 0, st, p);
      if (!p.fuse) hipLaunchKernelGGL(k_attn_combine<128>, cgrid, dim3(256), 0, st, p);
      break;
    case 64:
      if (two) hipLaunchKernelGGL((k_attn<64, 2>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_attn<64, 1>), grid, dim3(256), 0, st, p);
      if (!p.fuse) hipLaunchKernelGGL(k_attn_combine<64>, cgrid, dim3(256), 0, st, p);
      break;
    case 32:
      if (two) hipLaunchKernelGGL((k_attn<32, 2>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_attn<32, 1>), grid, dim3(256), 0, st, p);
      if (!p.fuse) hipLaunchKernelGGL(k_attn_combine<32>, cgrid, dim3(256), 0, st, p);
      break;
    case 16:
      if (two) hipLaunchKernelGGL((k_attn<16, 2>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_attn<16, 1>), grid, dim3(256), 0, st, p);
      if (!p.fuse) hipLaunchKernelGGL(k_attn_combine<16>, cgrid, dim3(256), 0, st, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedParams& p, int R, hipStream_t st) {
  if (R < 1 || p.S < 1 || R % p.S || !p.rowinfo || !p.slotbt || !p.seq_ids || !p.kv_len || !p.bt)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_embed, dim3(R), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const uint16_t* src, int rows, int cols, void* dst, int kind, int row0, int hd,
                            uint32_t* overflow, hipStream_t st) {
  if (!overflow) return hipErrorInvalidValue;
  const size_t total = (size_t)rows * (cols / 8);
  const int grid = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_pack_bf16, dim3(grid), dim3(256), 0, st, src, rows, cols, (u32x4*)dst, kind, row0, hd,
                     overflow);
  return hipGetLastError();
}

hipError_t launch_pack_int4(const uint8_t* q4, const uint16_t* scales, int rows, int cols, void* dst_frag,
                            uint16_t* dst_scales, int kind, int row0, int hd, hipStream_t st) {
  if (cols % 128) return hipErrorInvalidValue;
  const size_t total = (size_t)rows * (cols / 128);
  const int grid = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_pack_int4, dim3(grid), dim3(256), 0, st, q4, scales, rows, cols, (uint32_t*)dst_frag,
                     dst_scales, kind, row0, hd);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* dst, uint32_t value, size_t count, hipStream_t st) {
  if (count == 0) return hipSuccess;
  const int grid = (int)((count + 255) / 256 < 65535 ? (count + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_fill_u32, dim3(grid), dim3(256), 0, st, (uint32_t*)dst, value, count);
  return hipGetLastError();
}

}  // namespace specv
