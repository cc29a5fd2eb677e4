// forward.hip -- the verify forward as ONE persistent gfx950 kernel.
//
// One launch runs the whole trunk forward over the span rows (pegainfer page
// "DFlash speculative decoding", transaction section: one verify forward over
// [last, d1..dK] with the argmax of every row) and ends with accept_greedy
// and the cache advance.  The grid is exactly the set of workgroups the GPU
// holds at once (cooperative launch), and the forward's steps are phases:
//
//   embed | per layer: QKV(+RMSNorm, RoPE, KV write) | attention |
//           O(+residual) | gate/up(+RMSNorm, SwiGLU) | down(+residual) | LM head
//
// A phase may start once the previous phase's completion counter reaches its
// total (one count per finished 64-column block, attention head or row), so
// kernel boundaries and their cache flushes disappear.  Weights never depend
// on activations, so before waiting a workgroup already issues the weight
// fragment loads of its first unit of the next GEMM phase; the wait overlaps
// with the DRAM latency of that stream.
//
// Coherence: activations written in one phase and read in a later one cross
// XCDs (each XCD has its own L2), so they are stored and loaded with
// device-coherent (agent-scope) accesses; a producer waits for its stores to
// complete before it bumps a counter.  Weights are read-only for the whole
// launch and use plain non-temporal loads.
//
// Every wait is bounded: past the bound the launch records a watchdog error
// and every later wait returns at once, so every wave always exits.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace specv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef SPECV_POLL_SLEEP
#define SPECV_POLL_SLEEP 1  // s_sleep units (64 clocks) between two polls of a counter
#endif
constexpr unsigned kSpinLimit = (1u << 22) / SPECV_POLL_SLEEP;  // ~0.2 s of polling per wait

// ------------------------------------------------------ coherent accesses
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ldc2(const float* p) {  // 8-byte aligned
  const unsigned long long v =
      __hip_atomic_load((const unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc2(float* p, float a, float b) {  // 8-byte aligned
  const unsigned long long v = (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sth(_Float16* p, float v) {
  const _Float16 h = (_Float16)v;
  __hip_atomic_store((unsigned short*)p, __builtin_bit_cast(unsigned short, h), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 ldc16(const void* p) {  // 16 bytes as two coherent 8-byte loads
  const unsigned long long* q = (const unsigned long long*)p;
  const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (u32x4){(unsigned)a, (unsigned)(a >> 32), (unsigned)b, (unsigned)(b >> 32)};
}
__device__ __forceinline__ unsigned long long ldc8(const void* p) {
  return __hip_atomic_load((const unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

// --------------------------------------------------------- phase counters

// Block until done[ph] >= total (thread 0 polls; the workgroup then goes on).
__device__ __forceinline__ void wait_phase(const FwdParams& P, int ph, unsigned total) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    int ok = 1;
    while (__hip_atomic_load(P.done + ph, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < total) {
      if (__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ok = 0; break; }
      __builtin_amdgcn_s_sleep(SPECV_POLL_SLEEP);
      if (++spins > kSpinLimit) {
        atomicOr(P.err, 1);
        ok = 0;
        break;
      }
    }
    s_ok = ok;
    if (P.clock && blockIdx.x == 0) P.clock[ph] = __builtin_amdgcn_s_memrealtime();
  }
  __syncthreads();
  (void)s_ok;
}

// After this workgroup's stores for a finished item: make them visible, count it.
__device__ __forceinline__ void signal_phase(const FwdParams& P, int ph) {
  wait_all();
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(P.done + ph, 1u);
}

// ---------------------------------------------------------------- embed

__device__ __forceinline__ void embed_phase(const FwdParams& P, int wg, int G) {
  const int H = P.H, nb = H / 64;
  for (int r = wg; r < P.R; r += G) {
    const int tok = P.tokens[r];
    const uint16_t* e = P.emb + (size_t)tok * H;
    for (int c0 = 0; c0 < H; c0 += 256) {
      if (c0 + (int)(threadIdx.x & ~63) < H) {  // whole waves in or out
        const int c = c0 + threadIdx.x;
        const float v = __uint_as_float((uint32_t)e[c] << 16);
        stc(P.x + (size_t)r * H + c, v);
        float t = v * v;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
        if ((threadIdx.x & 63) == 0) stc(P.ss + (size_t)r * nb + c / 64, t);
      }
    }
    signal_phase(P, 0);
  }
}

// ------------------------------------------------------------ GEMM phases
//
// Y[R, N] = A'[R, K] W^T.  A unit is (64-column block nb, K slice s of NK*32
// inputs); wave w of the workgroup owns the 16-row weight tile 4*nb + w.  The
// ns slices of a column block belong to ns different workgroups; a workgroup
// keeps one slice for the whole phase (so A is staged into LDS once when
// R <= 16) and walks the column blocks nb = j, j + Gs, ...  Weights for the
// next unit are loaded while the current one computes.  The last slice of a
// column block to arrive sums the slices in slice order and runs the epilogue.

struct GemmPh {
  const u32x4* W;
  int N, K, ns;
  const float* A;   // [R][lda] activations (coherent loads)
  int lda;
  const float* ss;  // RMSNorm partial sums [R][ss_n] or null
  int ss_n;
  const float* gain;
  int ph;           // phase counter index
  int layer;
};

template <int NK>
__device__ __forceinline__ void issue_frags(u32x4 (&b)[NK], const GemmPh& g, int nb, int s) {
  const int tile = nb * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const u32x4* wp = g.W + ((size_t)tile * (g.K / 32) + (size_t)s * NK) * 64 + lane;
#pragma unroll
  for (int j = 0; j < NK; ++j) b[j] = __builtin_nontemporal_load(wp + j * 64);
}

// This workgroup's first unit of a GEMM phase, or nb = -1 if it has none.
__device__ __forceinline__ void first_unit(const GemmPh& g, int wg, int G, int& nb, int& s) {
  const int Gs = G / g.ns;
  nb = -1;
  s = 0;
  if (wg >= Gs * g.ns) return;
  s = wg % g.ns;
  const int j = wg / g.ns;
  if (j < (g.N >> 6)) nb = j;
}

// Stage rows m0..m0+15 of the slice into LDS in the MFMA A-operand order,
// RMSNorm applied, as bf16 hi + lo.
template <int NK>
__device__ __forceinline__ void stage_a(const FwdParams& P, const GemmPh& g, int s, int m0, u32x4* sA, float* sR) {
  const int tid = threadIdx.x;
  if (g.ss) {
    const int row = tid >> 4, part = tid & 15, r = m0 + row;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = part + 16 * i;
      v[i] = (r < P.R && q < g.ss_n) ? ldc(g.ss + (size_t)r * g.ss_n + q) : 0.0f;
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i];
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (part == 0) sR[row] = r < P.R ? 1.0f / sqrtf(acc * P.inv_dim + P.eps) : 0.0f;
    __syncthreads();
  }
  const int k0 = s * NK * 32;
  for (int u = tid; u < 16 * NK * 4; u += 256) {
    const int gq = u & 3, j = (u >> 2) % NK, row = u / (4 * NK);
    const int r = m0 + row;
    const int k = k0 + j * 32 + gq * 8;
    float v[8];
    if (r < P.R) {
      const float* src = g.A + (size_t)r * g.lda + k;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float2 t = ldc2(src + e);
        v[e] = t.x;
        v[e + 1] = t.y;
      }
      if (g.ss) {
        const float rs = sR[row];
        const f32x4 g0 = *(const f32x4*)(g.gain + k), g1 = *(const f32x4*)(g.gain + k + 4);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (v[e] * rs) * gg[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = (__bf16)v[e];
      hi[e] = h;
      lo[e] = (__bf16)(v[e] - (float)h);
    }
    const int l = gq * 16 + row;
    sA[(j * 2) * 64 + l] = __builtin_bit_cast(u32x4, hi);
    sA[(j * 2 + 1) * 64 + l] = __builtin_bit_cast(u32x4, lo);
  }
  __syncthreads();
}

constexpr int kMaxSlices = 32;  // K slices per GEMM (host-checked)

// Column pair (c, c+1) of row r summed over the K slices in slice order; all
// slice loads are issued before the first add (one memory round trip).
__device__ __forceinline__ void reduce_pair(const FwdParams& P, const GemmPh& g, int r, int c, float& v0, float& v1) {
  float2 t[kMaxSlices];
  const float* src = P.part + (size_t)r * g.N + c;
  const size_t stride = (size_t)P.R * g.N;
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s)
    if (s < g.ns) t[s] = ldc2(src + s * stride);
  v0 = 0.0f;
  v1 = 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s)
    if (s < g.ns) {
      v0 += t[s].x;
      v1 += t[s].y;
    }
}

__device__ __forceinline__ void row_pos(const FwdParams& P, int r, int& seq, int& pos) {
  const int b = r / P.S, i = r - b * P.S;
  seq = P.seq_ids[b];
  pos = P.kv_len[seq] + i;
}

template <int EPI>
__device__ __forceinline__ void epilogue(const FwdParams& P, const GemmPh& g, int nb, int* sArg);

template <>
__device__ __forceinline__ void epilogue<EPI_QKV>(const FwdParams& P, const GemmPh& g, int nb, int*) {
  const int hd = P.hd, half = hd / 2, DQ = P.DQ, DK = P.DK;
  _Float16* kpool = (_Float16*)(P.KV + (size_t)g.layer * P.kv_layer_bytes);
  _Float16* vpool = (_Float16*)(P.KV + (size_t)g.layer * P.kv_layer_bytes + P.kv_half_bytes);
  for (int idx = threadIdx.x; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float v0, v1;
    reduce_pair(P, g, r, c, v0, v1);
    int seq, pos;
    row_pos(P, r, seq, pos);
    const int blk = P.bt[(size_t)seq * P.bt_stride + (pos >> 4)], slot = pos & 15;
    if (c < DQ + DK) {  // the pair (d, d + hd/2) is stored interleaved
      const int local = c < DQ ? c : c - DQ;
      const int head = local / hd, j = (local % hd) >> 1;
      const float cs = P.rope[((size_t)pos * half + j) * 2], sn = P.rope[((size_t)pos * half + j) * 2 + 1];
      const float o0 = v0 * cs - v1 * sn, o1 = v0 * sn + v1 * cs;
      if (c < DQ) {
        float* qr = P.q + (size_t)r * DQ + head * hd;
        stc(qr + j, o0);
        stc(qr + j + half, o1);
      } else {
        _Float16* kr = kpool + (((size_t)blk * P.nkv + head) * 16 + slot) * hd;
        sth(kr + j, o0);
        sth(kr + j + half, o1);
      }
    } else {
      const int local = c - DQ - DK;
      const int head = local / hd, d = local % hd;
      _Float16* vb = vpool + ((size_t)blk * P.nkv + head) * hd * 16;
      sth(vb + (size_t)d * 16 + slot, v0);
      sth(vb + (size_t)(d + 1) * 16 + slot, v1);
    }
  }
}

template <>
__device__ __forceinline__ void epilogue<EPI_RESID>(const FwdParams& P, const GemmPh& g, int nb, int*) {
  const int NB = g.N >> 6;
  for (int idx = threadIdx.x; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float v0, v1;
    reduce_pair(P, g, r, c, v0, v1);
    float* xp = P.x + (size_t)r * g.N + c;
    const float2 x = ldc2(xp);
    const float x0 = x.x + v0, x1 = x.y + v1;
    stc2(xp, x0, x1);
    float t = x0 * x0 + x1 * x1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) t += __shfl_xor(t, o);
    if ((idx & 31) == 0) stc(P.ss + (size_t)r * NB + nb, t);
  }
}

template <>
__device__ __forceinline__ void epilogue<EPI_SWIGLU>(const FwdParams& P, const GemmPh& g, int nb, int*) {
  const int F = g.N >> 1;
  for (int idx = threadIdx.x; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float gt, up;
    reduce_pair(P, g, r, c, gt, up);
    stc(P.h + (size_t)r * F + (c >> 1), (gt / (1.0f + expf(-gt))) * up);
  }
}

template <>
__device__ __forceinline__ void epilogue<EPI_LM>(const FwdParams& P, const GemmPh& g, int nb, int*) {
  for (int idx = threadIdx.x; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float v0, v1;
    reduce_pair(P, g, r, c, v0, v1);
    if (P.logits) *(float2*)(P.logits + (size_t)r * g.N + c) = make_float2(v0, v1);
    if (v0 != v0 || v1 != v1) atomicOr(P.status, 1);
    const unsigned long long k0 = argmax_key(v0, c), k1 = argmax_key(v1, c + 1);
    unsigned long long k = k0 > k1 ? k0 : k1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      const unsigned long long t = __shfl_xor(k, o);
      k = t > k ? t : k;
    }
    if ((idx & 31) == 0) atomicMax(P.argkey + r, k);
  }
}

// Run by the workgroup that finishes the last LM column block: decode the
// row maxima, accept_greedy per sequence, advance the cache lengths.
__device__ __forceinline__ void accept_stage(const FwdParams& P, int* sArg) {
  for (int r = threadIdx.x; r < P.R; r += 256) {
    const unsigned long long k = atomicExch(P.argkey + r, 0ull);
    sArg[r] = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
  }
  __syncthreads();
  const int mode = P.step->mode, S = P.S;
  for (int b = threadIdx.x; b < P.n_seq; b += 256) {
    const int row0 = b * S;
    int m;
    if (mode == MODE_COMMIT_ALL) {
      m = S - 1;
    } else {
      m = 0;
      while (m < S - 1 && P.tokens[row0 + m + 1] == sArg[row0 + m]) ++m;
    }
    const int seq = P.seq_ids[b];
    if (mode == MODE_COMMIT_ALL) P.kv_len[seq] += S;
    else if (mode == MODE_VERIFY) P.kv_len[seq] += m + 1;
    int32_t* res = P.result + 1 + b * (S + 1);
    res[0] = m;
    for (int i = 0; i < S; ++i) res[1 + i] = sArg[row0 + i];
  }
  if (threadIdx.x == 0) {
    P.result[0] = atomicExch(P.status, 0) | (__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? 2 : 0);
    *P.lm_cnt = 0u;
    if (P.clock) P.clock[P.n_phases + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

// Run this workgroup's units of one GEMM phase.  `pre` holds the in-flight
// weight fragments of its first unit (issued before the phase's wait).
// Partial sums are written without waiting; once all units are issued the
// workgroup waits for its stores once, bumps the arrival counter of every
// column block it worked on, and runs the epilogue of each block it
// completed last.  No wait sits between two units, so the weight stream of
// the next unit overlaps the current unit's compute and stores.
template <int NK, int NKMAX, int EPI>
__device__ __forceinline__ void gemm_phase(const FwdParams& P, const GemmPh& g, u32x4 (&pre)[NKMAX], int wg, int G, char* smem) {
  int nb0, s;
  first_unit(g, wg, G, nb0, s);
  if (nb0 < 0) return;
  const int Gs = G / g.ns, NB = g.N >> 6;
  u32x4* sA = (u32x4*)smem;
  float* sR = (float*)(smem + NK * 2 * 64 * 16);
  int* sN = (int*)(sR + 16);  // [0] = count, then the column blocks completed last
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool once = P.R <= 16;
  if (once) stage_a<NK>(P, g, s, 0, sA, sR);
  u32x4 cur[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) cur[j] = pre[j];
  for (int nb = nb0; nb < NB; nb += Gs) {
    const int nxt = nb + Gs;
    u32x4 nx[NK];
    if (nxt < NB) {
      const int tile = nxt * 4 + wave;
      const u32x4* wp = g.W + ((size_t)tile * (g.K / 32) + (size_t)s * NK) * 64 + lane;
#pragma unroll
      for (int j = 0; j < NK; ++j) nx[j] = __builtin_nontemporal_load(wp + j * 64);
    }
    const int tile = nb * 4 + wave;
    for (int m0 = 0; m0 < P.R; m0 += 16) {
      if (!once) stage_a<NK>(P, g, s, m0, sA, sR);
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const bf16x8 bw = __builtin_bit_cast(bf16x8, cur[j]);
        const bf16x8 ah = __builtin_bit_cast(bf16x8, sA[(j * 2) * 64 + lane]);
        const bf16x8 al = __builtin_bit_cast(bf16x8, sA[(j * 2 + 1) * 64 + lane]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, acc, 0, 0, 0);
      }
      const int col = tile * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + (lane >> 4) * 4 + i;
        if (r < P.R) stc(P.part + ((size_t)s * P.R + r) * g.N + col, acc[i]);
      }
      if (!once) __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) cur[j] = nx[j];
  }
  wait_all();
  __syncthreads();
  if (tid == 0) sN[0] = 0;
  __syncthreads();
  // one arrival per column block, all issued at once (thread i: block i)
  for (int nb = nb0 + tid * Gs; nb < NB; nb += 256 * Gs)
    if (atomicAdd(P.cnt + nb, 1u) == (unsigned)(g.ns - 1)) {
      __hip_atomic_store(P.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sN[1 + atomicAdd(sN, 1)] = nb;
    }
  __syncthreads();
  const int n_last = sN[0];
  for (int i = 0; i < n_last; ++i) epilogue<EPI>(P, g, sN[1 + i], nullptr);
  if (n_last == 0) return;
  wait_all();
  __syncthreads();
  if (EPI == EPI_LM) {
    __shared__ int s_final;
    if (tid == 0) s_final = (atomicAdd(P.lm_cnt, (unsigned)n_last) + (unsigned)n_last == (unsigned)NB);
    __syncthreads();
    if (s_final) accept_stage(P, sN + 1);
  } else if (tid == 0) {
    atomicAdd(P.done + g.ph, (unsigned)n_last);
  }
}

// Issue the weight loads of this workgroup's first unit of phase g.
template <int NK, int NKMAX>
__device__ __forceinline__ void prefetch_phase(const GemmPh& g, u32x4 (&pre)[NKMAX], int wg, int G) {
  int nb, s;
  first_unit(g, wg, G, nb, s);
  if (nb < 0) return;
  u32x4 t[NK];
  issue_frags<NK>(t, g, nb, s);
#pragma unroll
  for (int j = 0; j < NK; ++j) pre[j] = t[j];
}

// -------------------------------------------------------------- attention
//
// Unit (256-key split, kv head, sequence).  One 64-key chunk per wave;
// scores are computed transposed (S^T = K Q^T) so the probabilities come out
// in the B-operand layout of O^T = V^T P^T.  Chunks combine in LDS in wave
// order, each split's (max, sum, o) goes to memory, and the last split of a
// (sequence, kv head) combines splits in split order.  Split and chunk
// boundaries are absolute positions.

template <int HD>
__device__ __forceinline__ void attn_unit(const FwdParams& P, int layer, int split, int kvh, int b, char* smem) {
  constexpr int KST = (HD + 31) / 32;
  constexpr int DT = HD / 16;
  const int seq = P.seq_ids[b];
  const int p = P.kv_len[seq];
  const int S = P.S, G = P.nq / P.nkv, QC = S * G;
  const int total = p + S;
  const int n_act = (total + 255) >> 8;
  if (split >= n_act) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int DQ = P.nq * HD;
  const _Float16* kpool = (const _Float16*)(P.KV + (size_t)layer * P.kv_layer_bytes);
  const _Float16* vpool = (const _Float16*)(P.KV + (size_t)layer * P.kv_layer_bytes + P.kv_half_bytes);

  float (*sO)[16][HD + 1] = (float (*)[16][HD + 1])smem;
  float* sM = (float*)(smem + 4 * 16 * (HD + 1) * 4);
  float* sL = sM + 64;
  float* sF = sL + 64;
  int* sLast = (int*)(sF + 64);

  const int kb0 = split * 16 + wave * 4;
  f16x8 kf[4][KST];
  f16x4 vf[4][DT];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kb = kb0 + t;
    const bool ok = kb * 16 < total;
    const int blk = ok ? P.bt[(size_t)seq * P.bt_stride + kb] : 0;
    const _Float16* kbase = kpool + ((size_t)blk * P.nkv + kvh) * 16 * HD;
    const _Float16* vbase = vpool + ((size_t)blk * P.nkv + kvh) * HD * 16;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const int d = ks * 32 + g4 * 8;
      if (ok && d < HD) kf[t][ks] = __builtin_bit_cast(f16x8, ldc16(kbase + c16 * HD + d));
      else kf[t][ks] = (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (ok) vf[t][dt] = __builtin_bit_cast(f16x4, ldc8(vbase + (dt * 16 + c16) * 16 + g4 * 4));
      else vf[t][dt] = (f16x4){0, 0, 0, 0};
    }
  }

  const int n_qt = (QC + 15) >> 4;
  for (int qt = 0; qt < n_qt; ++qt) {
    const int col = qt * 16 + c16;
    const bool qok = col < QC;
    const int iq = qok ? col / G : 0, hh = qok ? col % G : 0;
    const int head = kvh * G + hh;
    const int pos_q = p + iq;
    const float* qrow = P.q + (size_t)(b * S + iq) * DQ + head * HD;
    f16x8 qf[KST];
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const int d = ks * 32 + g4 * 8;
      f16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (qok && d < HD) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 t = ldc2(qrow + d + e);
          v[e] = (_Float16)t.x;
          v[e + 1] = (_Float16)t.y;
        }
      }
      qf[ks] = v;
    }
    float sc[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[t][ks], qf[ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = (kb0 + t) * 16 + g4 * 4 + i;
        sc[t][i] = (qok && key <= pos_q) ? acc[i] * P.scale : -INFINITY;
        mx = fmaxf(mx, sc[t][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float l = 0.0f;
    f16x8 pf[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = (mx == -INFINITY) ? 0.0f : expf(sc[t][i] - mx);
        l += e;
        pf[t >> 1][(t & 1) * 4 + i] = (_Float16)e;
      }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const f16x4 v0 = vf[2 * s2][dt], v1 = vf[2 * s2 + 1][dt];
        const f16x8 a = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[s2], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sO[wave][c16][dt * 16 + g4 * 4 + i] = acc[i];
    }
    if (g4 == 0) {
      sM[wave * 16 + c16] = mx;
      sL[wave * 16 + c16] = l;
    }
    __syncthreads();
    if (tid < 16) {
      const int c = tid;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sM[w * 16 + c]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = (M == -INFINITY) ? 0.0f : expf(sM[w * 16 + c] - M);
        sF[w * 16 + c] = f;
        L += sL[w * 16 + c] * f;
      }
      const int qcol = qt * 16 + c;
      if (qcol < QC) {
        float* dst = P.apart + (((size_t)kvh * P.max_splits + split) * (P.n_seq * QC) + b * QC + qcol) * (HD + 2);
        stc2(dst, M, L);
      }
    }
    __syncthreads();
    for (int e = tid; e < 16 * (HD / 2); e += 256) {
      const int c = e / (HD / 2), d = 2 * (e % (HD / 2));
      const int qcol = qt * 16 + c;
      if (qcol >= QC) continue;
      float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = sF[w * 16 + c];
        o0 += sO[w][c][d] * f;
        o1 += sO[w][c][d + 1] * f;
      }
      float* dst = P.apart + (((size_t)kvh * P.max_splits + split) * (P.n_seq * QC) + b * QC + qcol) * (HD + 2);
      stc2(dst + 2 + d, o0, o1);
    }
    __syncthreads();
  }

  wait_all();
  __syncthreads();
  if (tid == 0) *sLast = (atomicAdd(P.attn_cnt + b * P.nkv + kvh, 1u) == (unsigned)(n_act - 1));
  __syncthreads();
  if (!*sLast) return;
  if (tid == 0) __hip_atomic_store(P.attn_cnt + b * P.nkv + kvh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const size_t stride = (size_t)(P.n_seq * QC) * (HD + 2);
  const float* base = P.apart + ((size_t)kvh * P.max_splits * (P.n_seq * QC) + b * QC) * (HD + 2);
  float* sW = &sO[0][0][0];
  // (max, sum) of every (split, column) -> weights in LDS; loads in groups of 8
  for (int qcol = tid; qcol < QC; qcol += 256) {
    const int nsp = ((p + qcol / G) >> 8) + 1;
    float M = -INFINITY;
    for (int s0 = 0; s0 < nsp; s0 += 8) {
      float2 ml[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < nsp) ml[i] = ldc2(base + (s0 + i) * stride + (size_t)qcol * (HD + 2));
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < nsp) {
          M = fmaxf(M, ml[i].x);
          sW[(s0 + i) * QC + qcol] = ml[i].x;
          sW[(s0 + i) * QC + qcol + P.max_splits * QC] = ml[i].y;
        }
    }
    float L = 0.0f;
    for (int sp = 0; sp < nsp; ++sp) {
      const float f = expf(sW[sp * QC + qcol] - M);
      sW[sp * QC + qcol] = f;
      L += sW[sp * QC + qcol + P.max_splits * QC] * f;
    }
    for (int sp = 0; sp < nsp; ++sp) sW[sp * QC + qcol] /= L;
  }
  __syncthreads();
  for (int e = tid; e < QC * (HD / 2); e += 256) {
    const int qcol = e / (HD / 2), d = 2 * (e % (HD / 2));
    const int iq = qcol / G, head = kvh * G + qcol % G;
    const int nsp = ((p + iq) >> 8) + 1;
    const float* src = base + (size_t)qcol * (HD + 2) + 2 + d;
    float o0 = 0.0f, o1 = 0.0f;
    for (int s0 = 0; s0 < nsp; s0 += 8) {
      float2 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < nsp) v[i] = ldc2(src + (s0 + i) * stride);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < nsp) {
          const float f = sW[(s0 + i) * QC + qcol];
          o0 += v[i].x * f;
          o1 += v[i].y * f;
        }
    }
    stc2(P.o + (size_t)(b * S + iq) * DQ + head * HD + d, o0, o1);
  }
  signal_phase(P, 2 + 5 * layer);
}

template <int HD>
__device__ __forceinline__ void attn_phase(const FwdParams& P, int layer, int wg, int G, char* smem) {
  const int units = P.max_splits * P.nkv * P.n_seq;
  for (int u = wg; u < units; u += G) {
    const int split = u % P.max_splits, kvh = (u / P.max_splits) % P.nkv, b = u / (P.max_splits * P.nkv);
    attn_unit<HD>(P, layer, split, kvh, b, smem);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- kernel

__device__ __forceinline__ GemmPh make_ph(const FwdParams& P, int layer, int which) {
  GemmPh g;
  const uint8_t* lw = P.W + (size_t)layer * P.lay_stride;
  g.layer = layer;
  g.ss = nullptr;
  g.ss_n = P.H / 64;
  g.gain = nullptr;
  switch (which) {
    case 0:  // QKV
      g.W = (const u32x4*)(lw + P.off_wqkv); g.N = P.Nqkv; g.K = P.H; g.A = P.x; g.lda = P.H;
      g.ss = P.ss; g.gain = (const float*)(lw + P.off_gattn); g.ph = 1 + 5 * layer;
      break;
    case 1:  // O
      g.W = (const u32x4*)(lw + P.off_wo); g.N = P.H; g.K = P.DQ; g.A = P.o; g.lda = P.DQ; g.ph = 3 + 5 * layer;
      break;
    case 2:  // gate/up
      g.W = (const u32x4*)(lw + P.off_wgu); g.N = P.Ngu; g.K = P.H; g.A = P.x; g.lda = P.H;
      g.ss = P.ss; g.gain = (const float*)(lw + P.off_gffn); g.ph = 4 + 5 * layer;
      break;
    case 3:  // down
      g.W = (const u32x4*)(lw + P.off_wd); g.N = P.H; g.K = P.F; g.A = P.h; g.lda = P.F; g.ph = 5 + 5 * layer;
      break;
    default:  // LM head
      g.W = (const u32x4*)P.wlm; g.N = P.V; g.K = P.H; g.A = P.x; g.lda = P.H; g.ss = P.ss; g.gain = P.g_final;
      g.ph = 1 + 5 * P.L;
      break;
  }
  g.ns = g.K / (32 * (which == 1 ? P.nk_o : which == 3 ? P.nk_d : P.nk_h));
  return g;
}

template <int NKH, int NKO, int NKD, int HD>
__global__ __launch_bounds__(256) void k_forward(FwdParams P) {
  constexpr int NKMAX = NKH > NKO ? (NKH > NKD ? NKH : NKD) : (NKO > NKD ? NKO : NKD);
  constexpr int GEMM_LDS = NKMAX * 2 * 64 * 16 + 16 * 4 + (1 + 256) * 4;  // A tile, rstd, block list / row argmax
  constexpr int ATTN_LDS = 4 * 16 * (HD + 1) * 4 + 3 * 64 * 4 + 16;
  __shared__ __attribute__((aligned(16))) char smem[GEMM_LDS > ATTN_LDS ? GEMM_LDS : ATTN_LDS];
  const int wg = blockIdx.x, G = gridDim.x;
  const int H = P.H;
  if (P.clock && wg == 0 && threadIdx.x == 0) P.clock[P.n_phases] = __builtin_amdgcn_s_memrealtime();
  u32x4 pre[NKMAX];
  const unsigned nb_qkv = P.Nqkv / 64, nb_h = H / 64, nb_gu = P.Ngu / 64;
  const unsigned heads = (unsigned)(P.n_seq * P.nkv);

  embed_phase(P, wg, G);
  {  // the first layer's QKV weights load while the embedding finishes
    const GemmPh g = make_ph(P, 0, 0);
    prefetch_phase<NKH>(g, pre, wg, G);
  }
  for (int l = 0; l < P.L; ++l) {
    const GemmPh gq = make_ph(P, l, 0);
    wait_phase(P, l == 0 ? 0 : 5 * l, l == 0 ? (unsigned)P.R : nb_h);
    gemm_phase<NKH, NKMAX, EPI_QKV>(P, gq, pre, wg, G, smem);
    wait_phase(P, 1 + 5 * l, nb_qkv);
    attn_phase<HD>(P, l, wg, G, smem);
    const GemmPh go = make_ph(P, l, 1);
    prefetch_phase<NKO>(go, pre, wg, G);
    wait_phase(P, 2 + 5 * l, heads);
    gemm_phase<NKO, NKMAX, EPI_RESID>(P, go, pre, wg, G, smem);
    const GemmPh gu = make_ph(P, l, 2);
    prefetch_phase<NKH>(gu, pre, wg, G);
    wait_phase(P, 3 + 5 * l, nb_h);
    gemm_phase<NKH, NKMAX, EPI_SWIGLU>(P, gu, pre, wg, G, smem);
    const GemmPh gd = make_ph(P, l, 3);
    prefetch_phase<NKD>(gd, pre, wg, G);
    wait_phase(P, 4 + 5 * l, nb_gu);
    gemm_phase<NKD, NKMAX, EPI_RESID>(P, gd, pre, wg, G, smem);
    const GemmPh gn = (l + 1 < P.L) ? make_ph(P, l + 1, 0) : make_ph(P, 0, 4);
    prefetch_phase<NKH>(gn, pre, wg, G);
  }
  wait_phase(P, 5 * P.L, nb_h);
  gemm_phase<NKH, NKMAX, EPI_LM>(P, make_ph(P, 0, 4), pre, wg, G, smem);

  // Last workgroup out resets the phase counters for the next launch.
  __syncthreads();
  if (threadIdx.x == 0) {
    if (atomicAdd(P.exit_cnt, 1u) == (unsigned)(G - 1)) {
      for (int i = 0; i < P.n_phases; ++i) __hip_atomic_store(P.done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.exit_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int NKH, int NKO, int NKD, int HD>
hipError_t launch_fwd_t(const FwdParams& p, int grid, hipStream_t st) {
  void* args[] = {(void*)&p};
  return hipLaunchCooperativeKernel((const void*)k_forward<NKH, NKO, NKD, HD>, dim3(grid), dim3(256), args, 0, st);
}

template <int NKH, int NKO, int NKD, int HD>
int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)k_forward<NKH, NKO, NKD, HD>, 256, 0) != hipSuccess)
    return 0;
  return n;
}

}  // namespace

// Shapes with compiled forward kernels: (NK of K=hidden, NK of K=n_q*hd,
// NK of K=ffn, head_dim).  NK = inputs per K slice / 32.
#define SPECV_FWD_SHAPES(X) \
  X(16, 16, 16, 128)        \
  X(2, 2, 4, 16)

bool forward_supported(int nkh, int nko, int nkd, int hd) {
#define X(a, b, c, d) if (nkh == a && nko == b && nkd == c && hd == d) return true;
  SPECV_FWD_SHAPES(X)
#undef X
  return false;
}

int forward_occupancy(int nkh, int nko, int nkd, int hd) {
#define X(a, b, c, d) if (nkh == a && nko == b && nkd == c && hd == d) return occupancy_t<a, b, c, d>();
  SPECV_FWD_SHAPES(X)
#undef X
  return 0;
}

hipError_t launch_forward_kernel(const FwdParams& p, int grid, hipStream_t st) {
#define X(a, b, c, d) \
  if (p.nk_h == a && p.nk_o == b && p.nk_d == c && p.hd == d) return launch_fwd_t<a, b, c, d>(p, grid, st);
  SPECV_FWD_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace specv
