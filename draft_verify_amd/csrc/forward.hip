// forward.hip -- the verify forward as ONE persistent gfx950 kernel whose
// waves specialise.
//
// One launch runs the whole trunk forward over the span rows (pegainfer page
// "DFlash speculative decoding", transaction section: one verify forward over
// [last, d1..dK] with the argmax of every row) and ends with accept_greedy
// and the cache advance.  The grid is one 512-thread workgroup per CU, all
// co-resident (cooperative launch).  The forward's steps are phases:
//
//   embed | per layer: QKV(+RMSNorm, RoPE, KV write) | attention |
//           O(+residual) | gate/up(+RMSNorm, SwiGLU) | down(+residual) | LM head
//
// Roles.  Waves 0-3 of a workgroup are streamers: they walk the workgroup's
// GEMM units of every phase, in order, from the first layer's QKV to the LM
// head, with the weights of the next three units always in flight (a ring of
// three register buffers, so no load ever waits for a register copy), and
// run the MFMAs as soon as a unit's activation tile is staged.  Weights never
// depend on activations, so the weight stream runs through phase boundaries
// until the ring is full.  Waves 4-7 are helpers: they stage the activation
// tiles (RMSNorm, bf16 hi + lo) into LDS, move the streamers' 16x16 results
// from LDS to the split-K partial sums in memory, run the arrivals and
// epilogues, the embedding and the attention, and every cross-workgroup wait.
// The split matters on gfx9: a wave's memory counter is in order over loads
// and stores, so a poll or an epilogue load issued by a wave that has weight
// loads in flight would wait for them; helpers never have weight loads in
// flight, streamers never wait on memory other than their own weights.
//
// Hand-offs inside a workgroup go through LDS words written and read with
// workgroup-scope relaxed atomics (ds_write / ds_read, so no memory-counter
// waits); a wave's LDS operations complete in issue order, so a flag written
// after the data it guards is seen after that data.  The helpers synchronise
// among themselves with an LDS barrier of their own (the hardware barrier
// would need the streamers too).
//
// Across workgroups a phase may start once the previous phase's completion
// counter reaches its total (one count per finished 64-column block,
// attention head or row).  Activations written in one phase and read in a
// later one cross XCDs (each XCD has its own L2), so they are stored and
// loaded with device-coherent (agent-scope) accesses; a producer waits for
// its stores to complete before it bumps a counter.
//
// Every wait is bounded: past the bound the launch records a watchdog error,
// the workgroup marks itself aborted and every later wait returns at once, so
// every wave always exits.
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
typedef __attribute__((address_space(1))) u32x4 gu32x4;  // global memory, so loads stay off the LDS counter

// The unit table's per-workgroup index is read through the constant
// address space (scalar loads, read-only for the launch); the workgroup's
// own units are copied into LDS at launch, so the streamers read them with
// LDS loads instead of scalar loads whose waits would mix with the LDS
// counter.
typedef __attribute__((address_space(4))) const int32_t ci32;
__device__ __forceinline__ int unit_first(const FwdParams& P, int i) { return ((ci32*)P.unit_first)[i]; }

constexpr unsigned kSpinLimit = 1u << 22;  // polls (s_sleep 1 apart) before a wait gives up (~0.2-1 s)
constexpr int kSlices = 32;                // K slices per GEMM (host-checked)

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
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }  // lgkmcnt(0) only

__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

// ------------------------------------------------------------------- LDS

template <int NKMAX, int HD>
struct Lds {
  u32x4 A[2][NKMAX * 2 * 64];  // activation tiles of two consecutive GEMM phases (MFMA A order, hi/lo)
  f32x4 res[4][2][64];         // streamer s -> helper wave s: two 16x16 result slots
  float rstd[16];
  int list[1 + 256];           // column blocks completed last / row argmax for the accept stage
  float att_o[4][16][HD + 1];  // attention: per-wave chunk outputs, then the split-combine weights
  float att_m[64], att_l[64], att_f[64];
  int att_last;
  unsigned bar_arrive, bar_gen;  // helper barrier
  int a_ready[2];                // GEMM phase whose tile buffer k holds (-1: none yet)
  unsigned res_seq[4][2];        // (unit sequence number + 1) a streamer wrote into a slot
  unsigned res_ack[4][2];        // the same, after the helper wave read it
  int abort;                     // a wait of this workgroup gave up
  int ok;
  FwdUnit units[kFwdMaxWalk];    // this workgroup's walk, copied from the unit table at launch
};

__device__ __forceinline__ unsigned lds_ld(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_ld(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void cfence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

struct UnitInfo {
  uint64_t woff;
  uint32_t tile_stride;
  int g, nk, nb, sl;
};
// Unit i of this workgroup's walk (LDS copy).
template <class S>
__device__ __forceinline__ UnitInfo unit_at(const S& s, int i) {
  const FwdUnit& u = s.units[i];
  UnitInfo r;
  r.woff = u.woff;
  r.tile_stride = u.tile_stride;
  r.g = u.g;
  r.nk = u.nk;
  r.nb = u.nb;
  r.sl = u.sl;
  return r;
}

// Give up on a wait: record the watchdog error and abort this workgroup.
template <class S>
__device__ __forceinline__ void give_up(const FwdParams& P, S& s) {
  lds_st(&s.abort, 1);
  atomicOr(P.err, 1);
}

// Spin until *p == want (an LDS word), bounded.
template <class S, class T>
__device__ __forceinline__ void spin_eq(const FwdParams& P, S& s, const T* p, T want) {
  unsigned spins = 0;
  while (lds_ld(p) != want) {
    if (lds_ld(&s.abort)) break;
    if (++spins > kSpinLimit) {
      give_up(P, s);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  cfence();
}

// Barrier of the four helper waves (LDS arrival count + generation).
template <class S>
__device__ __forceinline__ void hbar(const FwdParams& P, S& s) {
  wait_lds();
  cfence();
  if ((threadIdx.x & 63) == 0) {
    const unsigned g = lds_ld(&s.bar_gen);
    if (__hip_atomic_fetch_add(&s.bar_arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 3u) {
      lds_st(&s.bar_arrive, 0u);
      lds_st(&s.bar_gen, g + 1u);
    } else {
      unsigned spins = 0;
      while (lds_ld(&s.bar_gen) == g) {
        if (++spins > kSpinLimit) {  // never expected: helpers only wait on bounded waits
          give_up(P, s);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  cfence();
}

// --------------------------------------------------------- phase counters

// Helpers: block until done[ph] >= total (helper thread 0 polls).
template <class S>
__device__ __forceinline__ void wait_phase(const FwdParams& P, S& s, int ht, int ph, unsigned total) {
  if (ht == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(P.done + ph, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < total) {
      if (lds_ld(&s.abort) || __hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        lds_st(&s.abort, 1);
        break;
      }
      if (++spins > kSpinLimit) {
        give_up(P, s);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (P.clock && blockIdx.x == 0) P.clock[ph] = __builtin_amdgcn_s_memrealtime();
  }
  hbar(P, s);
}

// Helpers, after the stores of finished items: make them visible, count n.
template <class S>
__device__ __forceinline__ void signal_phase(const FwdParams& P, S& s, int ht, int ph, unsigned n) {
  wait_all();
  hbar(P, s);
  if (ht == 0 && n) atomicAdd(P.done + ph, n);
}

// ------------------------------------------------------------ GEMM phases
//
// GEMM phase g: 4l + {0 QKV, 1 O, 2 gate/up, 3 down} for layer l, 4L = LM
// head.  Y[R, N] = A'[R, K] W^T.  A unit is (64-column block nb, K slice sl
// of nk*32 inputs); streamer wave w takes the 16-column tile 4*nb + w.
// Workgroup wg keeps slice wg % ns for the whole phase (so the activation
// tile is staged once) and walks the blocks wg / ns + k * (G / ns).

struct Phase {
  const u32x4* W;
  int N, K, nk, ns, sl, j0, Gs, NB, n;  // n: this workgroup's units
  int which, layer;
};

__device__ __forceinline__ Phase phase_of(const FwdParams& P, int g, int wg, int G) {
  Phase ph;
  const int l = g >> 2, which = (g >= 4 * P.L) ? 4 : (g & 3);
  const uint8_t* lw = P.W + (size_t)(which == 4 ? 0 : l) * P.lay_stride;
  ph.which = which;
  ph.layer = which == 4 ? P.L : l;
  switch (which) {
    case 0: ph.W = (const u32x4*)(lw + P.off_wqkv); ph.N = P.Nqkv; ph.K = P.H; ph.nk = P.nk_h; break;
    case 1: ph.W = (const u32x4*)(lw + P.off_wo); ph.N = P.H; ph.K = P.DQ; ph.nk = P.nk_o; break;
    case 2: ph.W = (const u32x4*)(lw + P.off_wgu); ph.N = P.Ngu; ph.K = P.H; ph.nk = P.nk_h; break;
    case 3: ph.W = (const u32x4*)(lw + P.off_wd); ph.N = P.H; ph.K = P.F; ph.nk = P.nk_d; break;
    default: ph.W = (const u32x4*)P.wlm; ph.N = P.V; ph.K = P.H; ph.nk = P.nk_h; break;
  }
  ph.ns = ph.K / (32 * ph.nk);
  ph.Gs = G / ph.ns;
  ph.NB = ph.N >> 6;
  ph.sl = wg % ph.ns;
  ph.j0 = wg / ph.ns;
  ph.n = (wg < ph.Gs * ph.ns && ph.j0 < ph.NB) ? (ph.NB - ph.j0 + ph.Gs - 1) / ph.Gs : 0;
  return ph;
}

// Issue this wave's weight loads of unit U into B (NKMAX loads always, so
// the memory counter sees the same count per unit; steps past the slice
// reload its last fragment; past the walk's end, the arena's first
// fragment).  The base is wave-uniform and lives in scalar registers.
template <int NKMAX, class S>
__device__ __forceinline__ void issue(const FwdParams& P, const S& s, int u, int n, u32x4 (&B)[NKMAX], int sw, int lane) {
  uint64_t base = (uint64_t)P.W;
  int last = 0;
  if (u < n) {
    const UnitInfo U = unit_at(s, u);
    base += U.woff + (uint64_t)sw * U.tile_stride;
    last = U.nk - 1;
  }
#pragma unroll
  for (int j = 0; j < NKMAX; ++j) {
    const uint64_t pj = base + (uint64_t)(j < last ? j : last) * 1024;
    // readfirstlane returns a signed int: widen each half as unsigned
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(pj >> 32));
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pj);
    const gu32x4* q = (const gu32x4*)((hi << 32) | lo);
    B[j] = __builtin_nontemporal_load(q + lane);
  }
}

// One unit's MFMAs once its activation tile is staged; the 16x16 result goes
// to this wave's LDS slot for the helper wave of the same index.
template <int NKMAX, class S>
__device__ __forceinline__ void consume(const FwdParams& P, S& s, const u32x4 (&B)[NKMAX], unsigned useq, int sw,
                                        int lane) {
  const UnitInfo U = unit_at(s, (int)useq);
  const int g = U.g, nk = U.nk;
  spin_eq(P, s, &s.a_ready[g & 1], g);
  const u32x4* A = s.A[g & 1];
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < NKMAX; ++j) {
    if (j < nk) {
      const bf16x8 bw = __builtin_bit_cast(bf16x8, B[j]);
      const bf16x8 ah = __builtin_bit_cast(bf16x8, A[(j * 2) * 64 + lane]);
      const bf16x8 al = __builtin_bit_cast(bf16x8, A[(j * 2 + 1) * 64 + lane]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, acc, 0, 0, 0);
    }
  }
  const int slot = useq & 1;
  if (useq >= 2) spin_eq(P, s, &s.res_ack[sw][slot], useq - 1);
  s.res[sw][slot][lane] = acc;
  cfence();
  lds_st(&s.res_seq[sw][slot], useq + 1);
}

// The streamer walk: every GEMM unit of this workgroup, three in flight.
template <int NKMAX, class S>
__device__ __forceinline__ void streamer(const FwdParams& P, S& s, int wg) {
  const int sw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int NP = 4 * P.L + 2;
  const int n = unit_first(P, wg * NP + NP - 1) - unit_first(P, wg * NP);
  u32x4 B0[NKMAX], B1[NKMAX], B2[NKMAX];
  issue<NKMAX>(P, s, 0, n, B0, sw, lane);
  issue<NKMAX>(P, s, 1, n, B1, sw, lane);
  issue<NKMAX>(P, s, 2, n, B2, sw, lane);
  for (int u = 0; u < n; u += 3) {
    consume<NKMAX>(P, s, B0, (unsigned)u, sw, lane);
    issue<NKMAX>(P, s, u + 3, n, B0, sw, lane);
    if (u + 1 >= n) break;
    consume<NKMAX>(P, s, B1, (unsigned)(u + 1), sw, lane);
    issue<NKMAX>(P, s, u + 4, n, B1, sw, lane);
    if (u + 2 >= n) break;
    consume<NKMAX>(P, s, B2, (unsigned)(u + 2), sw, lane);
    issue<NKMAX>(P, s, u + 5, n, B2, sw, lane);
  }
  wait_all();  // the trailing loads land before the wave exits
}

// --------------------------------------------------------------- helpers

__device__ __forceinline__ void row_pos(const FwdParams& P, int r, int& seq, int& pos) {
  const int b = r / P.S, i = r - b * P.S;
  seq = P.seq_ids[b];
  pos = P.kv_len[seq] + i;
}

// The embedding rows of this workgroup: x = E[token] in fp32 plus the sum of
// squares of every 64-column block.
template <class S>
__device__ __forceinline__ void embed_phase(const FwdParams& P, S& s, int ht, int wg, int G) {
  const int H = P.H, nb = H / 64;
  for (int r = wg; r < P.R; r += G) {
    const int tok = P.tokens[r];
    const uint16_t* e = P.emb + (size_t)tok * H;
    for (int c0 = 0; c0 < H; c0 += 256) {
      if (c0 + (ht & ~63) < H) {  // whole waves in or out
        const int c = c0 + ht;
        const float v = __uint_as_float((uint32_t)e[c] << 16);
        stc(P.x + (size_t)r * H + c, v);
        float t = v * v;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
        if ((ht & 63) == 0) stc(P.ss + (size_t)r * nb + c / 64, t);
      }
    }
    signal_phase(P, s, ht, 0, 1u);
  }
}

// Stage rows 0..15 of the phase's slice into LDS buffer g & 1 in the MFMA
// A-operand order, RMSNorm applied (QKV, gate/up, LM), as bf16 hi + lo; then
// tell the streamers.
template <int NKMAX, class S>
__device__ __forceinline__ void stage_a(const FwdParams& P, S& s, int ht, int g, const Phase& ph) {
  const float* A;
  int lda;
  const float* gain = nullptr;
  const uint8_t* lw = P.W + (size_t)(ph.which == 4 ? 0 : ph.layer) * P.lay_stride;
  switch (ph.which) {
    case 0: A = P.x; lda = P.H; gain = (const float*)(lw + P.off_gattn); break;
    case 1: A = P.o; lda = P.DQ; break;
    case 2: A = P.x; lda = P.H; gain = (const float*)(lw + P.off_gffn); break;
    case 3: A = P.h; lda = P.F; break;
    default: A = P.x; lda = P.H; gain = P.g_final; break;
  }
  const int ss_n = P.H / 64;
  if (gain) {
    const int row = ht >> 4, part = ht & 15;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = part + 16 * i;
      v[i] = (row < P.R && q < ss_n) ? ldc(P.ss + (size_t)row * ss_n + q) : 0.0f;
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i];
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (part == 0) s.rstd[row] = row < P.R ? 1.0f / sqrtf(acc * P.inv_dim + P.eps) : 0.0f;
    hbar(P, s);
  }
  u32x4* sA = s.A[g & 1];
  const int NK = ph.nk, k0 = ph.sl * NK * 32;
  for (int u = ht; u < 16 * NK * 4; u += 256) {
    const int gq = u & 3, j = (u >> 2) % NK, row = u / (4 * NK);
    const int k = k0 + j * 32 + gq * 8;
    float v[8];
    if (row < P.R) {
      const float* src = A + (size_t)row * lda + k;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float2 t = ldc2(src + e);
        v[e] = t.x;
        v[e + 1] = t.y;
      }
      if (gain) {
        const float rs = s.rstd[row];
        const f32x4 g0 = *(const f32x4*)(gain + k), g1 = *(const f32x4*)(gain + k + 4);
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
  hbar(P, s);
  if (ht == 0) lds_st(&s.a_ready[g & 1], g);
}

// Column pair (c, c+1) of row r summed over the K slices in slice order; all
// slice loads are issued before the first add.
__device__ __forceinline__ void reduce_pair(const FwdParams& P, const Phase& ph, int r, int c, float& v0, float& v1) {
  float2 t[kSlices];
  const float* src = P.part + (size_t)r * ph.N + c;
  const size_t stride = (size_t)P.R * ph.N;
#pragma unroll
  for (int q = 0; q < kSlices; ++q)
    if (q < ph.ns) t[q] = ldc2(src + q * stride);
  v0 = 0.0f;
  v1 = 0.0f;
#pragma unroll
  for (int q = 0; q < kSlices; ++q)
    if (q < ph.ns) {
      v0 += t[q].x;
      v1 += t[q].y;
    }
}

__device__ __forceinline__ void epi_qkv(const FwdParams& P, const Phase& ph, int nb, int ht) {
  const int hd = P.hd, half = hd / 2, DQ = P.DQ, DK = P.DK;
  _Float16* kpool = (_Float16*)(P.KV + (size_t)ph.layer * P.kv_layer_bytes);
  _Float16* vpool = (_Float16*)(P.KV + (size_t)ph.layer * P.kv_layer_bytes + P.kv_half_bytes);
  for (int idx = ht; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float v0, v1;
    reduce_pair(P, ph, r, c, v0, v1);
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

__device__ __forceinline__ void epi_resid(const FwdParams& P, const Phase& ph, int nb, int ht) {
  const int NB = ph.N >> 6;
  for (int idx = ht; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float v0, v1;
    reduce_pair(P, ph, r, c, v0, v1);
    float* xp = P.x + (size_t)r * ph.N + c;
    const float2 x = ldc2(xp);
    const float x0 = x.x + v0, x1 = x.y + v1;
    stc2(xp, x0, x1);
    float t = x0 * x0 + x1 * x1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) t += __shfl_xor(t, o);
    if ((idx & 31) == 0) stc(P.ss + (size_t)r * NB + nb, t);
  }
}

__device__ __forceinline__ void epi_swiglu(const FwdParams& P, const Phase& ph, int nb, int ht) {
  const int F = ph.N >> 1;
  for (int idx = ht; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float gt, up;
    reduce_pair(P, ph, r, c, gt, up);
    stc(P.h + (size_t)r * F + (c >> 1), (gt / (1.0f + expf(-gt))) * up);
  }
}

__device__ __forceinline__ void epi_lm(const FwdParams& P, const Phase& ph, int nb, int ht) {
  for (int idx = ht; idx < P.R * 32; idx += 256) {
    const int r = idx >> 5, c = nb * 64 + 2 * (idx & 31);
    float v0, v1;
    reduce_pair(P, ph, r, c, v0, v1);
    if (P.logits) *(float2*)(P.logits + (size_t)r * ph.N + c) = make_float2(v0, v1);
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

// Run by the helpers of the workgroup that finishes the last LM column
// block: decode the row maxima, accept_greedy per sequence, advance the
// cache lengths.
template <class S>
__device__ __forceinline__ void accept_stage(const FwdParams& P, S& s, int ht) {
  int* arg = s.list + 1;
  for (int r = ht; r < P.R; r += 256) {
    const unsigned long long k = atomicExch(P.argkey + r, 0ull);
    arg[r] = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
  }
  hbar(P, s);
  const int mode = P.step->mode, S_ = P.S;
  for (int b = ht; b < P.n_seq; b += 256) {
    const int row0 = b * S_;
    int m;
    if (mode == MODE_COMMIT_ALL) {
      m = S_ - 1;
    } else {
      m = 0;
      while (m < S_ - 1 && P.tokens[row0 + m + 1] == arg[row0 + m]) ++m;
    }
    const int seq = P.seq_ids[b];
    if (mode == MODE_COMMIT_ALL) P.kv_len[seq] += S_;
    else if (mode == MODE_VERIFY) P.kv_len[seq] += m + 1;
    int32_t* res = P.result + 1 + b * (S_ + 1);
    res[0] = m;
    for (int i = 0; i < S_; ++i) res[1 + i] = arg[row0 + i];
  }
  if (ht == 0) {
    P.result[0] = atomicExch(P.status, 0) | (__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? 2 : 0);
    *P.lm_cnt = 0u;
    if (P.clock) P.clock[P.n_phases + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

// Helpers' side of one GEMM phase: stage its tile, move the streamers'
// results to the split partial sums as they come, then one arrival per
// column block (all at once) and the epilogue of every block this
// workgroup completed last.
template <int NKMAX, int EPI, class S>
__device__ __forceinline__ void helper_gemm(const FwdParams& P, S& s, int ht, int g, int wg, int G, int done_ph) {
  Phase ph = phase_of(P, g, wg, G);
  const int NP = 4 * P.L + 2;
  const int ubase = unit_first(P, wg * NP);     // the walk's first unit
  const int k0 = unit_first(P, wg * NP + g);    // this phase's units in the table
  ph.n = unit_first(P, wg * NP + g + 1) - k0;
  if (ph.n) {
    ph.sl = unit_at(s, k0 - ubase).sl;
    stage_a<NKMAX>(P, s, ht, g, ph);
  }
  const int hw = ht >> 6, lane = ht & 63;
  for (int k = 0; k < ph.n; ++k) {
    const unsigned useq = (unsigned)(k0 - ubase + k);
    const int slot = useq & 1;
    spin_eq(P, s, &s.res_seq[hw][slot], useq + 1);
    const f32x4 acc = s.res[hw][slot][lane];
    cfence();
    lds_st(&s.res_ack[hw][slot], useq + 1);
    const int nb = unit_at(s, k0 - ubase + k).nb;
    const int col = (nb * 4 + hw) * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (lane >> 4) * 4 + i;
      if (r < P.R) stc(P.part + ((size_t)ph.sl * P.R + r) * ph.N + col, acc[i]);
    }
  }
  wait_all();
  hbar(P, s);
  if (ht == 0) lds_st(&s.list[0], 0);
  hbar(P, s);
  for (int k = ht; k < ph.n; k += 256) {
    const int nb = unit_at(s, k0 - ubase + k).nb;
    if (atomicAdd(P.cnt + nb, 1u) == (unsigned)(ph.ns - 1)) {
      __hip_atomic_store(P.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s.list[1 + __hip_atomic_fetch_add(&s.list[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)] = nb;
    }
  }
  hbar(P, s);
  const int n_last = lds_ld(&s.list[0]);
  for (int i = 0; i < n_last; ++i) {
    const int nb = s.list[1 + i];
    if (EPI == EPI_QKV) epi_qkv(P, ph, nb, ht);
    else if (EPI == EPI_RESID) epi_resid(P, ph, nb, ht);
    else if (EPI == EPI_SWIGLU) epi_swiglu(P, ph, nb, ht);
    else epi_lm(P, ph, nb, ht);
  }
  if (EPI == EPI_LM) {
    wait_all();
    hbar(P, s);
    if (n_last) {
      if (ht == 0) s.ok = (atomicAdd(P.lm_cnt, (unsigned)n_last) + (unsigned)n_last == (unsigned)ph.NB);
      hbar(P, s);
      if (s.ok) accept_stage(P, s, ht);
    }
  } else {
    signal_phase(P, s, ht, done_ph, (unsigned)n_last);
  }
}

// -------------------------------------------------------------- attention
//
// Unit (256-key split, kv head, sequence) on the four helper waves.  One
// 64-key chunk per wave; scores are computed transposed (S^T = K Q^T) so the
// probabilities come out in the B-operand layout of O^T = V^T P^T.  Chunks
// combine in LDS in wave order, each split's (max, sum, o) goes to memory,
// and the last split of a (sequence, kv head) combines splits in split
// order.  Split and chunk boundaries are absolute positions.

template <int HD, class S>
__device__ __forceinline__ void attn_unit(const FwdParams& P, S& s, int ht, int layer, int split, int kvh, int b) {
  constexpr int KST = (HD + 31) / 32;
  constexpr int DT = HD / 16;
  const int seq = P.seq_ids[b];
  const int p = P.kv_len[seq];
  const int S_ = P.S, G = P.nq / P.nkv, QC = S_ * G;
  const int total = p + S_;
  const int n_act = (total + 255) >> 8;
  if (split >= n_act) return;
  const int wave = ht >> 6, lane = ht & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int DQ = P.nq * HD;
  const _Float16* kpool = (const _Float16*)(P.KV + (size_t)layer * P.kv_layer_bytes);
  const _Float16* vpool = (const _Float16*)(P.KV + (size_t)layer * P.kv_layer_bytes + P.kv_half_bytes);

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
    const float* qrow = P.q + (size_t)(b * S_ + iq) * DQ + head * HD;
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
      for (int i = 0; i < 4; ++i) s.att_o[wave][c16][dt * 16 + g4 * 4 + i] = acc[i];
    }
    if (g4 == 0) {
      s.att_m[wave * 16 + c16] = mx;
      s.att_l[wave * 16 + c16] = l;
    }
    hbar(P, s);
    if (ht < 16) {
      const int c = ht;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s.att_m[w * 16 + c]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = (M == -INFINITY) ? 0.0f : expf(s.att_m[w * 16 + c] - M);
        s.att_f[w * 16 + c] = f;
        L += s.att_l[w * 16 + c] * f;
      }
      const int qcol = qt * 16 + c;
      if (qcol < QC) {
        float* dst = P.apart + (((size_t)kvh * P.max_splits + split) * (P.n_seq * QC) + b * QC + qcol) * (HD + 2);
        stc2(dst, M, L);
      }
    }
    hbar(P, s);
    for (int e = ht; e < 16 * (HD / 2); e += 256) {
      const int c = e / (HD / 2), d = 2 * (e % (HD / 2));
      const int qcol = qt * 16 + c;
      if (qcol >= QC) continue;
      float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = s.att_f[w * 16 + c];
        o0 += s.att_o[w][c][d] * f;
        o1 += s.att_o[w][c][d + 1] * f;
      }
      float* dst = P.apart + (((size_t)kvh * P.max_splits + split) * (P.n_seq * QC) + b * QC + qcol) * (HD + 2);
      stc2(dst + 2 + d, o0, o1);
    }
    hbar(P, s);
  }

  wait_all();
  hbar(P, s);
  if (ht == 0) s.att_last = (atomicAdd(P.attn_cnt + b * P.nkv + kvh, 1u) == (unsigned)(n_act - 1));
  hbar(P, s);
  if (!s.att_last) return;
  if (ht == 0) __hip_atomic_store(P.attn_cnt + b * P.nkv + kvh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const size_t stride = (size_t)(P.n_seq * QC) * (HD + 2);
  const float* base = P.apart + ((size_t)kvh * P.max_splits * (P.n_seq * QC) + b * QC) * (HD + 2);
  float* sW = &s.att_o[0][0][0];
  // (max, sum) of every (split, column) -> weights in LDS; loads in groups of 8
  for (int qcol = ht; qcol < QC; qcol += 256) {
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
  hbar(P, s);
  for (int e = ht; e < QC * (HD / 2); e += 256) {
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
    stc2(P.o + (size_t)(b * S_ + iq) * DQ + head * HD + d, o0, o1);
  }
  signal_phase(P, s, ht, 2 + 5 * layer, 1u);
}

template <int HD, class S>
__device__ __forceinline__ void attn_phase(const FwdParams& P, S& s, int ht, int layer, int wg, int G) {
  const int units = P.max_splits * P.nkv * P.n_seq;
  for (int u = wg; u < units; u += G) {
    const int split = u % P.max_splits, kvh = (u / P.max_splits) % P.nkv, b = u / (P.max_splits * P.nkv);
    attn_unit<HD>(P, s, ht, layer, split, kvh, b);
    hbar(P, s);
  }
}

template <int NKMAX, int HD, class S>
__device__ __forceinline__ void helpers(const FwdParams& P, S& s, int wg, int G) {
  const int ht = threadIdx.x - 256;
  const unsigned nb_qkv = P.Nqkv / 64, nb_h = P.H / 64, nb_gu = P.Ngu / 64;
  const unsigned heads = (unsigned)(P.n_seq * P.nkv);
  embed_phase(P, s, ht, wg, G);
  for (int l = 0; l < P.L; ++l) {
    wait_phase(P, s, ht, l == 0 ? 0 : 5 * l, l == 0 ? (unsigned)P.R : nb_h);
    helper_gemm<NKMAX, EPI_QKV>(P, s, ht, 4 * l, wg, G, 1 + 5 * l);
    wait_phase(P, s, ht, 1 + 5 * l, nb_qkv);
    attn_phase<HD>(P, s, ht, l, wg, G);
    wait_phase(P, s, ht, 2 + 5 * l, heads);
    helper_gemm<NKMAX, EPI_RESID>(P, s, ht, 4 * l + 1, wg, G, 3 + 5 * l);
    wait_phase(P, s, ht, 3 + 5 * l, nb_h);
    helper_gemm<NKMAX, EPI_SWIGLU>(P, s, ht, 4 * l + 2, wg, G, 4 + 5 * l);
    wait_phase(P, s, ht, 4 + 5 * l, nb_gu);
    helper_gemm<NKMAX, EPI_RESID>(P, s, ht, 4 * l + 3, wg, G, 5 + 5 * l);
  }
  wait_phase(P, s, ht, 5 * P.L, nb_h);
  helper_gemm<NKMAX, EPI_LM>(P, s, ht, 4 * P.L, wg, G, 0);
}

// ---------------------------------------------------------------- kernel

template <int NKH, int NKO, int NKD, int HD>
__global__ __launch_bounds__(512) void k_forward(FwdParams P) {
  constexpr int NKMAX = NKH > NKO ? (NKH > NKD ? NKH : NKD) : (NKO > NKD ? NKO : NKD);
  __shared__ Lds<NKMAX, HD> s;
  const int wg = blockIdx.x, G = gridDim.x;
  if (threadIdx.x == 0) {
    s.bar_arrive = 0u;
    s.bar_gen = 0u;
    s.a_ready[0] = -1;
    s.a_ready[1] = -1;
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 2; ++j) {
        s.res_seq[i][j] = 0u;
        s.res_ack[i][j] = 0u;
      }
    s.abort = 0;
    if (P.clock && wg == 0) P.clock[P.n_phases] = __builtin_amdgcn_s_memrealtime();
  }
  {
    const int NP = 4 * P.L + 2;
    const int u0 = unit_first(P, wg * NP), n = unit_first(P, wg * NP + NP - 1) - u0;
    for (int i = threadIdx.x; i < n; i += 512) s.units[i] = P.units[u0 + i];  // host-checked: n <= kFwdMaxWalk
  }
  __syncthreads();  // the only barrier of all eight waves
  if (threadIdx.x < 256) {
    streamer<NKMAX>(P, s, wg);
    return;
  }
  helpers<NKMAX, HD>(P, s, wg, G);
  // Last workgroup out resets the phase counters for the next launch.
  if (threadIdx.x == 256) {
    if (atomicAdd(P.exit_cnt, 1u) == (unsigned)(G - 1)) {
      for (int i = 0; i < P.n_phases; ++i) __hip_atomic_store(P.done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.exit_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int NKH, int NKO, int NKD, int HD>
hipError_t launch_fwd_t(const FwdParams& p, int grid, hipStream_t st) {
  void* args[] = {(void*)&p};
  return hipLaunchCooperativeKernel((const void*)k_forward<NKH, NKO, NKD, HD>, dim3(grid), dim3(512), args, 0, st);
}

template <int NKH, int NKO, int NKD, int HD>
int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)k_forward<NKH, NKO, NKD, HD>, 512, 0) != hipSuccess)
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
