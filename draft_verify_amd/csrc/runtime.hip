// runtime.hip -- host side of libspecv: buffer layout, weight packing, KV
// block management, the launch sequence of one forward, HIP graphs per
// (sequences, span) shape, and the C ABI of include/specv.h.
//
// Everything that changes between steps (span tokens, step mode, sequence
// ids, cache lengths, block tables) lives in device memory, so a graph
// captured once per exact shape is replayed unchanged; a graph is never
// replayed at a shape other than the one it was captured at.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <map>
#include <new>
#include <string>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/specv.h"
#include "internal.h"

using namespace specv;

static_assert(kMaxRows == SPEC_MAX_ROWS, "kernel row limit must match the ABI");

namespace {

thread_local std::string g_create_error;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Inputs per K slice for a GEMM of depth K: the largest of 512/256/128/64
// dividing K.  Fixed per (N, K), independent of the row count.
inline int slice_steps(int K) {
  for (int nk : {16, 8, 4, 2})
    if (K % (nk * 32) == 0) return nk;
  return 0;
}

// The many-row GEMM (bf16, above 16 rows, prepared A): the fewest K slices,
// each a whole number of its pipeline rounds, that give SPECV_BIG_WGS
// workgroups (one per CU; measured at 128 rows, more slices cost more in
// partial sums and their gather than they gain in balance: the 4B gate/up
// runs one slice and no gather); the LM head one slice, since its accept
// stage wants whole rows.  0: the shape does not fit the kernel.  Fixed per
// (N, K), whatever the rows.
#ifndef SPECV_BIG_WGS
#define SPECV_BIG_WGS 256
#endif
#ifndef SPECV_BIG_CT
#define SPECV_BIG_CT 1
#endif
inline int big_slices(int N, int K, int epi) {
  const int ct = SPECV_BIG_CT, pd = ct == 2 ? SPECV_BIG_PD2 : SPECV_BIG_PD1;
  if (K % 32 || N < 1) return 0;
  const int KS = K / 32, NB = (N + 64 * ct - 1) / (64 * ct);
  if (epi == EPI_LM) return KS % pd ? 0 : 1;
  if (N % 16) return 0;  // k_gather's groups of 8 pairs
  int best = 0;
  for (int ns = 1; ns <= KS; ++ns) {
    if (KS % ns || (KS / ns) % pd) continue;
    best = ns;
    if ((long long)NB * ns >= SPECV_BIG_WGS) break;
  }
  return best;
}

// int4: slices hold whole 128-input groups (16, 8 or 4 steps).
inline int slice_steps_int4(int K) {
  for (int nk : {16, 8, 4})
    if (K % (nk * 32) == 0) return nk;
  return 0;
}

// Which int4 kernel serves a GEMM of depth K (split-K slices of nk steps) at
// R rows; both the forward and the workspace sizing ask this one function.
// Depths whose register-activation plan is one K part run the one-pass LDS
// kernel with that plan's K parts up to eight rows (INT4_MMQ at depth *nk_mmq)
// and the register kernel from nine to sixteen rows (INT4_MMQR): the two add
// the same parts in the same order, so rows stay bit-exact across the switch.
// A depth the LDS kernel serves at its own parts (several register parts: O)
// keeps the LDS kernel up to eight rows and the split-K kernel, which adds
// those parts in that order, above; a depth it cannot serve (down) runs the
// register kernel for every R up to sixteen (several parts end in the residual
// epilogue's part sum; other epilogues keep the split-K kernel there).
enum { INT4_SPLITK = 0, INT4_MMQ = 1, INT4_MMQR = 2 };
inline int int4_route(int K, int nk, int R, int epi, int* nk_mmq) {
  int nw = 0, gpw = 0, parts = 0;
  const bool qr = mmqr_plan(K, &nw, &gpw, &parts);
  *nk_mmq = nk;
  if (R > 16) return INT4_SPLITK;
  if (qr && parts == 1) {
    if (R <= 8 && mmq_supported(K, 4 * gpw, epi)) {
      *nk_mmq = 4 * gpw;
      return INT4_MMQ;
    }
    return INT4_MMQR;
  }
  if (R <= 8 && mmq_supported(K, nk, epi)) return INT4_MMQ;
  if (qr && epi == EPI_RESID && !mmq_supported(K, nk, epi)) return INT4_MMQR;
  return INT4_SPLITK;
}

struct LayerOff {
  size_t wqkv, wo, wgu, wd, g_attn, g_ffn;
};

// One-pass GEMM plan of one projection (launch_mm): nw K parts of spw steps;
// nbuf 1 or 2: walking blocks of ct tiles with nbuf weight buffers; nbuf 0:
// one tile per workgroup loaded in ct phases; used for R <= rmax, so one
// kernel serves every R <= rmax and a row's result does not depend on the
// other rows (the rows gate).  Above rmax the split-K kernel runs with the
// depth that suits many rows; its results agree to rounding, not bit for bit.
// nw == 0 means the split-K kernel serves every R.
struct MmPlan {
  int nw, spw, ct, nbuf, gp, rmax;
};

// The down projection at K = 9728 for up to four rows: one tile per
// workgroup, 16 K parts of 19 steps, A staged in LDS (launch_mm1l); k_mm1
// with the same parts for up to SPECV_DOWN_MM1_ROWS rows, and the split-K
// kernel with the same parts (nk = 19) for more.

// Preference lists, first match on K = nw * spw * 32 wins.
#ifndef SPECV_MM_QKV
#define SPECV_MM_QKV {16, 5, 1, 1, 16, 16}, {1, 2, 1, 1, 1, 16}, {2, 1, 1, 1, 2, 16}
#endif
#ifndef SPECV_MM_GU
#define SPECV_MM_GU {16, 5, 1, 1, 16, 16}, {1, 2, 1, 1, 1, 16}, {2, 1, 1, 1, 2, 16}
#endif
#ifndef SPECV_MM_O
#define SPECV_MM_O {8, 16, 2, 0, 1, 8}, {16, 8, 1, 0, 1, 16}, {1, 2, 1, 1, 1, 16}, {2, 1, 1, 1, 2, 16}, {4, 1, 1, 1, 4, 16}
#endif
#ifndef SPECV_MM_LM
#define SPECV_MM_LM {16, 5, 1, 1, 16, 16}, {1, 2, 1, 1, 1, 16}, {2, 1, 1, 1, 2, 16}
#endif
#ifndef SPECV_MM_D
#define SPECV_MM_D {16, 8, 1, 0, 1, 16}, {1, 4, 1, 1, 1, 16}, {2, 2, 1, 1, 2, 16}, {1, 2, 1, 1, 1, 16}, {4, 1, 1, 1, 4, 16}
#endif

#ifndef SPECV_DOWN_LDS
#define SPECV_DOWN_LDS 1
#endif
#ifndef SPECV_O_LDS
#define SPECV_O_LDS 1
#endif
// Rows above four and up to this many take the down projection's one-pass
// kernel with A read from global memory (the same K parts, summed in the same
// order as the LDS-staged kernel); more rows take split-K.
#ifndef SPECV_DOWN_MM1_ROWS
#define SPECV_DOWN_MM1_ROWS 8
#endif
// Longest context, in 256-key splits, whose attention merges in k_attn.
#ifndef SPECV_ATTN_FUSE_SPLITS
#define SPECV_ATTN_FUSE_SPLITS 8
#endif
// Attention workgroups (sequence, kv head, split, query tile) up to which each
// takes one query tile.
#ifndef SPECV_ATTN_TPW1_WGS
#define SPECV_ATTN_TPW1_WGS 512
#endif
#ifndef SPECV_MM_WG_PER_CU
#define SPECV_MM_WG_PER_CU 1
#endif

MmPlan pick_mm(int epi, int K, std::initializer_list<MmPlan> prefs) {
  for (const MmPlan& m : prefs)
    if (m.nw * m.spw * 32 == K && mm_supported(epi, m.nw, m.spw, m.ct, m.nbuf, m.gp)) return m;
  return MmPlan{0, 0, 0, 0, 0, 0};
}

// Byte layout of the three device buffers for one description.
struct Layout {
  int fmt;  // FMT_BF16 or FMT_INT4 (GEMM weights; the embedding is bf16)
  int H, nq, nkv, hd, F, V, L, DQ, DK, Nqkv, Ngu;
  int max_rows, max_seqs, max_ctx, bt_stride, n_blocks, max_splits, G;
  int nk_qkv, nk_o, nk_gu, nk_d, nk_lm;
  MmPlan mm_qkv, mm_o, mm_gu, mm_d, mm_lm;  // per-kernel path, bf16: the one-pass GEMMs for R <= rmax
  bool d_lds;                        // down: the LDS-staged one-pass GEMM for R <= 4
  // weights
  std::vector<LayerOff> lay;
  size_t emb, wlm, g_final, weights_bytes;
  // kv
  // per layer: its K region at kv_off[l], V at kv_off[l] + kv_half[l]; a
  // global layer holds the paged pool, a sliding-window layer one ring of
  // ring_nb blocks per sequence
  std::vector<size_t> kv_off, kv_half;
  std::vector<char> local;   // per layer: sliding-window layer
  std::vector<char> rec;     // per layer: recurrent layer (its region holds the state snapshots)
  int win, ring_nb, ring_w, win_splits;
  bool any_rec;
  size_t kv_bytes;
  // workspace
  size_t af;  // prepared A of the split-K GEMMs above 16 rows (bf16), or (size_t)-1
  size_t af2; // the same for O and down, written by their producers
  size_t rowinfo;  // per row: position and KV block, written by k_embed
  size_t rec_kv, rec_slot;  // recurrent layers: staged keys and values; committed state slot per sequence
  size_t slotbt;   // per batch slot: its sequence's block table row, written by k_embed
  size_t x, ss, q, q16, o, h, part, cnt, attn_cnt, lm_cnt, packflag, h16, o16, argkey, status, step, result, kv_len, bt, rope, apart,
      logits, workspace_bytes;
  size_t host_step, host_result, host_kvlen, host_bt, host_bytes;
  int cnt_n;
};

inline size_t mat_bytes(int fmt, int N, int K) {
  return fmt == FMT_INT4 ? packed_int4_bytes(N, K) : packed_bf16_bytes(N, K);
}

bool build_layout(const spec_model_desc& d, Layout& Lo, std::string& err) {
  auto fail = [&](const char* m) {
    err = m;
    return false;
  };
  if (d.n_layers <= 0 || d.hidden <= 0 || d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.ffn <= 0 || d.vocab <= 0)
    return fail("model dimensions must be positive");
  if (d.weight_format != SPEC_WFMT_BF16 && d.weight_format != SPEC_WFMT_INT4G128)
    return fail("weight_format must be SPEC_WFMT_BF16 or SPEC_WFMT_INT4G128");
  Lo.fmt = d.weight_format == SPEC_WFMT_INT4G128 ? FMT_INT4 : FMT_BF16;
  if (Lo.fmt == FMT_INT4 && (d.hidden % 128 || d.ffn % 128 || (d.n_q_heads * d.head_dim) % 128))
    return fail("int4 group-128 weights need hidden, ffn and n_q_heads*head_dim multiples of 128");
  if (!(d.head_dim == 16 || d.head_dim == 32 || d.head_dim == 64 || d.head_dim == 128))
    return fail("head_dim must be 16, 32, 64 or 128");
  if (d.n_q_heads % d.n_kv_heads) return fail("n_q_heads must be a multiple of n_kv_heads");
  if (d.hidden % 64 || d.ffn % 32 || d.vocab % 64) return fail("hidden and vocab must be multiples of 64, ffn of 32");
  if (d.hidden > 8192) return fail("hidden must be at most 8192");
  if ((d.n_q_heads * d.head_dim) % 64 || ((d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim) % 64)
    return fail("attention projection widths must be multiples of 64");
  if (d.max_rows < 1 || d.max_rows > SPEC_MAX_ROWS) return fail("max_rows must be in [1, 128]");
  if (d.max_ctx < 1 || d.max_seqs < 1) return fail("max_ctx and max_seqs must be positive");
  if (!(d.rms_eps >= 0.0f) || !(d.rope_theta > 0.0)) return fail("rms_eps must be >= 0 and rope_theta > 0");
  if (d.swa_window < 0 || d.reserved != 0) return fail("swa_window must be >= 0 and reserved 0");
  if (d.swa_window > 0 && (d.swa_layers == 0 || (d.n_layers < 64 && (d.swa_layers >> d.n_layers) != 0)))
    return fail("swa_layers must name at least one existing layer when swa_window > 0");
  if (d.reserved2 != 0) return fail("reserved2 must be 0");
  if (d.rec_layers) {
    if (d.n_layers < 64 && (d.rec_layers >> d.n_layers) != 0) return fail("rec_layers names a layer past n_layers");
    if (d.swa_window > 0 && (d.rec_layers & d.swa_layers)) return fail("a layer cannot be both recurrent and windowed");
    if (!(d.rec_beta > 0.0f) || d.rec_beta > 1.0f) return fail("rec_beta must be in (0, 1]");
    if (d.n_q_heads / d.n_kv_heads > 8) return fail("recurrent layers take at most 8 query heads per kv head");
  }
  Lo.H = d.hidden; Lo.nq = d.n_q_heads; Lo.nkv = d.n_kv_heads; Lo.hd = d.head_dim; Lo.F = d.ffn; Lo.V = d.vocab;
  Lo.L = d.n_layers;
  Lo.DQ = Lo.nq * Lo.hd; Lo.DK = Lo.nkv * Lo.hd; Lo.Nqkv = Lo.DQ + 2 * Lo.DK; Lo.Ngu = 2 * Lo.F;
  Lo.G = Lo.nq / Lo.nkv;
  Lo.max_rows = d.max_rows; Lo.max_seqs = d.max_seqs; Lo.max_ctx = d.max_ctx;
  Lo.bt_stride = (d.max_ctx + SPEC_BLOCK_TOKENS - 1) / SPEC_BLOCK_TOKENS;
  Lo.n_blocks = d.n_blocks > 0 ? d.n_blocks : d.max_seqs * Lo.bt_stride;
  Lo.max_splits = (d.max_ctx + 255) / 256;
  auto steps = [&](int K) { return Lo.fmt == FMT_INT4 ? slice_steps_int4(K) : slice_steps(K); };
  Lo.nk_qkv = steps(Lo.H); Lo.nk_o = steps(Lo.DQ); Lo.nk_gu = Lo.nk_qkv;
  Lo.nk_d = steps(Lo.F);
  // The split-K LM head serves int4 above its one-pass rows (~10^4
  // workgroups, where half-depth slices keep more of them resident) and, in
  // bf16 above 16 rows, only shapes the many-row GEMM does not fit, with
  // full-depth slices (half the split partials, R x vocab x 4 bytes each).
  Lo.nk_lm = Lo.fmt == FMT_BF16 ? Lo.nk_qkv : std::min(Lo.nk_qkv, 8);
  if (Lo.fmt == FMT_INT4 && Lo.nk_lm % 4) Lo.nk_lm = Lo.nk_qkv;
  // int4 rows up to eight take the one-pass kernel at the QKV depth; more rows
  // keep the same K parts
  if (Lo.fmt == FMT_INT4 && mmq_supported(Lo.H, Lo.nk_qkv, EPI_LM)) Lo.nk_lm = Lo.nk_qkv;
  if (!Lo.nk_qkv || !Lo.nk_o || !Lo.nk_d) return fail("GEMM depths must be multiples of 64");
  Lo.mm_qkv = Lo.mm_o = Lo.mm_gu = Lo.mm_d = Lo.mm_lm = MmPlan{0, 0, 0, 0, 0, 0};
  Lo.d_lds = false;
  if (Lo.fmt == FMT_BF16) {
    // one-pass GEMMs for R <= 16; the split-K kernel (R > 16) then takes the
    // same K parts (nk = spw), so both give identical results
    Lo.mm_qkv = pick_mm(EPI_QKV, Lo.H, {SPECV_MM_QKV});
    Lo.mm_gu = pick_mm(EPI_SWIGLU, Lo.H, {SPECV_MM_GU});
    Lo.mm_o = pick_mm(EPI_RESID, Lo.DQ, {SPECV_MM_O});
    Lo.mm_d = pick_mm(EPI_RESID, Lo.F, {SPECV_MM_D});
    Lo.mm_lm = pick_mm(EPI_LM, Lo.H, {SPECV_MM_LM});
    // one-pass plans of R up to 16 that the split-K kernel cannot take at its
    // own depth keep their parts there too (rmax < 16: both serve R <= 16)
    if (SPECV_DOWN_LDS && !Lo.mm_d.nw && Lo.F == 16 * 19 * 32) {
      Lo.d_lds = true;
      Lo.nk_d = 19;
    }
    if (Lo.mm_qkv.nw && Lo.mm_qkv.rmax < 16) Lo.nk_qkv = Lo.mm_qkv.spw;
    if (Lo.mm_gu.nw && Lo.mm_gu.rmax < 16) Lo.nk_gu = Lo.mm_gu.spw;
    if (Lo.mm_o.nw && Lo.mm_o.rmax < 16) Lo.nk_o = Lo.mm_o.spw;
    if (Lo.mm_d.nw && Lo.mm_d.rmax < 16) Lo.nk_d = Lo.mm_d.spw;
    if (Lo.mm_lm.nw && Lo.mm_lm.rmax < 16) Lo.nk_lm = Lo.mm_lm.spw;
  }
  if (Lo.F % 64) return fail("ffn must be a multiple of 64");
  // the split merge holds up to 256 split weights per query column
  if (Lo.max_splits > 256) return fail("max_ctx must be at most 65536");

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  Lo.lay.resize((size_t)Lo.L);
  for (auto& l : Lo.lay) {
    l.wqkv = take(mat_bytes(Lo.fmt, Lo.Nqkv, Lo.H));
    l.wo = take(mat_bytes(Lo.fmt, Lo.H, Lo.DQ));
    l.wgu = take(mat_bytes(Lo.fmt, Lo.Ngu, Lo.H));
    l.wd = take(mat_bytes(Lo.fmt, Lo.H, Lo.F));
    l.g_attn = take((size_t)Lo.H * 4);
    l.g_ffn = take((size_t)Lo.H * 4);
  }
  Lo.emb = take((size_t)Lo.V * Lo.H * 2);
  Lo.wlm = take(mat_bytes(Lo.fmt, Lo.V, Lo.H));
  Lo.g_final = take((size_t)Lo.H * 4);
  Lo.weights_bytes = off;

  // Sliding-window layers keep a ring of ring_w = W + 16 slots (rounded up
  // to whole blocks) per sequence: a verify of at most 16 rows writes its rows
  // at their slots (position mod ring_w) without touching any position that
  // it, or any later query after a partial rejection, still attends to, so no
  // row ever needs restoring.
  Lo.win = d.swa_window;
  Lo.local.assign((size_t)Lo.L, 0);
  if (Lo.win > 0)
    for (int l = 0; l < Lo.L && l < 64; ++l) Lo.local[(size_t)l] = (d.swa_layers >> l) & 1u ? 1 : 0;
  Lo.ring_w = Lo.win > 0 ? (Lo.win + SPEC_MAX_SPAN + 15) / 16 * 16 : 0;
  Lo.ring_nb = Lo.ring_w / 16;
  // splits of 256 keys one row group's window can touch
  Lo.win_splits = Lo.win > 0 ? std::min(Lo.max_splits, (Lo.win + SPEC_MAX_SPAN - 1 + 255) / 256 + 1) : 0;
  // Recurrent layers keep no cache rows: their region holds, per sequence, two
  // sets of per-row state snapshots (one committed, one for the next forward).
  Lo.rec.assign((size_t)Lo.L, 0);
  Lo.any_rec = false;
  for (int l = 0; l < Lo.L && l < 64; ++l)
    if ((d.rec_layers >> l) & 1u) {
      Lo.rec[(size_t)l] = 1;
      Lo.any_rec = true;
    }
  Lo.kv_off.resize((size_t)Lo.L);
  Lo.kv_half.resize((size_t)Lo.L);
  Lo.kv_bytes = 0;
  for (int l = 0; l < Lo.L; ++l) {
    Lo.kv_off[(size_t)l] = Lo.kv_bytes;
    if (Lo.rec[(size_t)l]) {
      Lo.kv_half[(size_t)l] = 0;
      Lo.kv_bytes += align_up((size_t)Lo.max_seqs * 2 * SPEC_MAX_SPAN * Lo.nkv * Lo.hd * Lo.hd * 4);
      continue;
    }
    const size_t blocks = Lo.local[(size_t)l] ? (size_t)Lo.max_seqs * Lo.ring_nb : (size_t)Lo.n_blocks;
    Lo.kv_half[(size_t)l] = align_up(blocks * Lo.nkv * SPEC_BLOCK_TOKENS * Lo.hd * 2);
    Lo.kv_bytes += 2 * Lo.kv_half[(size_t)l];
  }

  const size_t R = (size_t)Lo.max_rows;
  off = 0;
  Lo.x = take(R * Lo.H * 4);
  Lo.ss = take(R * (Lo.H / 16) * 4);
  Lo.q = take(R * Lo.DQ * 4);
  Lo.q16 = take(R * Lo.DQ * 2);
  Lo.o = take(R * Lo.DQ * 4);
  Lo.h = take(R * Lo.F * 4);
  // Split partial sums, for the GEMMs that run the split-K kernel at some row
  // count up to max_rows (above the row limit of their one-pass kernel).
  // int4 GEMMs up to 16 rows run the register-activation one-pass kernel;
  // with several K parts (residual epilogues) its split buffer holds parts x N
  // per row
  size_t part = 0;
  auto onepass_rows = [&](const MmPlan& m, int K, int nk, int N, int epi) {
    if (m.nw) return std::min(m.rmax, 16);
    if (Lo.fmt != FMT_INT4) return 0;
    int lim = 0, nk_mmq = 0;
    for (int r = 1; r <= 16; ++r) {
      const int route = int4_route(K, nk, r, epi, &nk_mmq);
      if (route == INT4_SPLITK) break;
      lim = r;
      int nw = 0, gpw = 0, parts = 0;
      if (route == INT4_MMQR && mmqr_plan(K, &nw, &gpw, &parts) && parts > 1)
        part = std::max(part, (size_t)parts * N);
    }
    return lim;
  };
  const int lim_d = Lo.d_lds ? SPECV_DOWN_MM1_ROWS : onepass_rows(Lo.mm_d, Lo.F, Lo.nk_d, Lo.H, EPI_RESID);
  // Row counts above a GEMM's one-pass limit `lim` and at most 16 run the
  // split-K kernel (its nk-deep slices); above 16, bf16 runs the many-row
  // GEMM where the shape fits it (its slices' partials, none for one slice),
  // int4 and the shapes it does not fit the split-K kernel.  A description
  // can take both (up to 16 rows per sequence, more over a batch), so the
  // buffer holds the larger.
  auto need = [&](int lim, int N, int K, int nk, int epi) {
    const size_t split = (size_t)(K / (nk * 32)) * N;
    if (std::min(Lo.max_rows, 16) > lim) part = std::max(part, split);
    if (Lo.max_rows > 16) {
      const int ns = Lo.fmt == FMT_BF16 ? big_slices(N, K, epi) : 0;
      part = std::max(part, ns ? (ns > 1 ? (size_t)ns * N : (size_t)0) : split);
    }
  };
  need(onepass_rows(Lo.mm_qkv, Lo.H, Lo.nk_qkv, Lo.Nqkv, EPI_QKV), Lo.Nqkv, Lo.H, Lo.nk_qkv, EPI_QKV);
  need(onepass_rows(Lo.mm_o, Lo.DQ, Lo.nk_o, Lo.H, EPI_RESID), Lo.H, Lo.DQ, Lo.nk_o, EPI_RESID);
  need(onepass_rows(Lo.mm_gu, Lo.H, Lo.nk_gu, Lo.Ngu, EPI_SWIGLU), Lo.Ngu, Lo.H, Lo.nk_gu, EPI_SWIGLU);
  need(lim_d, Lo.H, Lo.F, Lo.nk_d, EPI_RESID);
  need(onepass_rows(Lo.mm_lm, Lo.H, Lo.nk_lm, Lo.V, EPI_LM), Lo.V, Lo.H, Lo.nk_lm, EPI_LM);
  Lo.part = take(std::max(part * R * 4, (size_t)256));
  Lo.cnt_n = std::max({Lo.Nqkv, Lo.H, Lo.Ngu, Lo.V}) / 64;
  Lo.cnt_n = std::max(Lo.cnt_n, Lo.H / 16);  // one per 16-column block of a residual GEMM
  Lo.cnt = take((size_t)Lo.cnt_n * 4);
  Lo.attn_cnt = take(R * Lo.nq * 4);  // n_seq * n_kv * query tiles <= rows * n_q
  Lo.lm_cnt = take(4);
  Lo.packflag = take(4);
  // fp16 copies of the SwiGLU and attention outputs for the one-pass down
  // and O kernels (at most 8 rows)
  Lo.h16 = take((size_t)std::min(R, (size_t)16) * Lo.F * 2);
  Lo.o16 = take((size_t)std::min(R, (size_t)16) * Lo.DQ * 2);
  Lo.rowinfo = take(R * 8);
  Lo.rec_kv = Lo.any_rec ? take(R * 2 * Lo.DK * 4) : (size_t)-1;
  Lo.rec_slot = Lo.any_rec ? take((size_t)Lo.max_seqs * 4) : (size_t)-1;
  Lo.slotbt = take((size_t)Lo.max_seqs * Lo.bt_stride * 4);
  Lo.argkey = take(R * 8);
  Lo.status = take(4);
  Lo.step = take(sizeof(StepDev) + 3 * R * 4);
  Lo.result = take((1 + 2 * R) * 4);
  Lo.kv_len = take((size_t)Lo.max_seqs * 4);
  Lo.bt = take((size_t)Lo.max_seqs * Lo.bt_stride * 4);
  Lo.rope = take((size_t)Lo.max_ctx * (Lo.hd / 2) * 2 * 4);
  Lo.apart = take((size_t)Lo.nkv * Lo.max_splits * R * Lo.G * (Lo.hd + 2) * 4);
  Lo.logits = (d.flags & SPEC_FLAG_KEEP_LOGITS) ? take(R * Lo.V * 4) : (size_t)-1;
  // prepared A (fp16, rows padded to 16)
  Lo.af = (Lo.fmt == FMT_BF16 && R > 16)
              ? take((R + 15) / 16 * 16 * (size_t)std::max({Lo.H, Lo.DQ, Lo.F}) * 2)
              : (size_t)-1;
  Lo.af2 = Lo.af != (size_t)-1 ? take((R + 15) / 16 * 16 * (size_t)std::max(Lo.DQ, Lo.F) * 2) : (size_t)-1;
  Lo.workspace_bytes = off;

  off = 0;
  Lo.host_step = take(sizeof(StepDev) + 3 * R * 4);
  Lo.host_result = take((1 + 2 * R) * 4);
  Lo.host_kvlen = take((size_t)Lo.max_seqs * 8);  // cache lengths, then recurrent slots
  Lo.host_bt = take((size_t)Lo.max_seqs * Lo.bt_stride * 4);
  Lo.host_bytes = off;
  return true;
}

}  // namespace

struct spec_ctx {
  spec_model_desc d;
  Layout lo;
  hipStream_t st;
  uint8_t *W, *KV, *WS, *HB;
  // host mirrors
  std::vector<int> len, nblk;
  std::vector<char> live;
  std::vector<int> free_blocks;
  std::vector<unsigned> loaded;  // bit per matrix/norm slot
  std::map<std::pair<int, int>, hipGraphExec_t> graphs;
  spec_stats stats;
  std::string err;
  int last_rows = 0;
  int mm_grid = 1;       // most workgroups of a one-pass GEMM (they walk the column blocks)
  int attn_fuse = 0;     // the current step's contexts are short: attention combines in one kernel
  int attn_tpw = 1;      // the current step's query tiles per attention workgroup
  int attn_fuse_l = 0, attn_tpw_l = 1;  // the same for the sliding-window layers
  hipEvent_t ev0 = nullptr, ev1 = nullptr;  // verify forward timing (spec_get_stats)
  int static_dev = -1;   // spec_create_static: the device whose scratch is the workspace
  float temp = 0.0f;     // spec_set_sampling: 0 greedy, > 0 sampled rows
  uint64_t seed = 0;

  template <class T> T* ws(size_t off) { return (T*)(WS + off); }
  void* af() { return lo.af == (size_t)-1 ? nullptr : (void*)(WS + lo.af); }
  // the prepared A that a producer writes for the residual GEMM (N outputs,
  // depth K) after it (O after attention, down after gate/up), or null when
  // that GEMM is not the many-row one and reads its fp32 A
  void* af_next(int N, int K, int R) {
    return lo.af2 != (size_t)-1 && R > 16 && big_slices(N, K, EPI_RESID) ? (void*)(WS + lo.af2) : nullptr;
  }
  int32_t* h_step() { return (int32_t*)(HB + lo.host_step); }
  int32_t* h_result() { return (int32_t*)(HB + lo.host_result); }
  int32_t* h_kvlen() { return (int32_t*)(HB + lo.host_kvlen); }
  int32_t* h_bt() { return (int32_t*)(HB + lo.host_bt); }
  _Float16* kpool(int l) { return (_Float16*)(KV + lo.kv_off[(size_t)l]); }
  _Float16* vpool(int l) { return (_Float16*)(KV + lo.kv_off[(size_t)l] + lo.kv_half[(size_t)l]); }
};

namespace {

int set_err(spec_ctx* c, int code, const std::string& m) {
  c->err = m;
  return code;
}

#define HIPCHK(ctx, call)                                                                    \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess) return set_err((ctx), SPEC_EHIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

// Slots of the loaded bitmap: 9 per layer (Q, K, V, O, GATE, UP, DOWN, norm a, norm f) + 3 globals.
int slot(const spec_ctx* c, int layer, int which) { return layer * 9 + which; }
int n_slots(const spec_ctx* c) { return c->lo.L * 9 + 3; }
bool all_loaded(const spec_ctx* c) {
  for (int i = 0; i < n_slots(c); ++i)
    if (!c->loaded[(size_t)i]) return false;
  return true;
}

// ---------------------------------------------------------------- blocks

int ensure_blocks(spec_ctx* c, int seq, int need_len, bool* dirty) {
  const int need = (need_len + SPEC_BLOCK_TOKENS - 1) / SPEC_BLOCK_TOKENS;
  while (c->nblk[(size_t)seq] < need) {
    if (c->free_blocks.empty()) return set_err(c, SPEC_ECAPACITY, "KV block pool exhausted");
    const int blk = c->free_blocks.back();
    c->free_blocks.pop_back();
    c->h_bt()[(size_t)seq * c->lo.bt_stride + c->nblk[(size_t)seq]] = blk;
    c->nblk[(size_t)seq]++;
    *dirty = true;
  }
  return SPEC_OK;
}

// Return blocks wholly past `len` to the pool, last allocated first.
void trim_blocks(spec_ctx* c, int seq, int len) {
  const int keep = (len + SPEC_BLOCK_TOKENS - 1) / SPEC_BLOCK_TOKENS;
  while (c->nblk[(size_t)seq] > keep) {
    c->nblk[(size_t)seq]--;
    c->free_blocks.push_back(c->h_bt()[(size_t)seq * c->lo.bt_stride + c->nblk[(size_t)seq]]);
  }
}

int upload_bt_row(spec_ctx* c, int seq) {
  const size_t o = (size_t)seq * c->lo.bt_stride;
  HIPCHK(c, hipMemcpyAsync(c->ws<int32_t>(c->lo.bt) + o, c->h_bt() + o, (size_t)c->lo.bt_stride * 4,
                           hipMemcpyHostToDevice, c->st));
  return SPEC_OK;
}

int upload_kv_len(spec_ctx* c, int seq) {
  c->h_kvlen()[seq] = c->len[(size_t)seq];
  HIPCHK(c, hipMemcpyAsync(c->ws<int32_t>(c->lo.kv_len) + seq, c->h_kvlen() + seq, 4, hipMemcpyHostToDevice, c->st));
  return SPEC_OK;
}

// A sequence that starts over (prefill, release) starts from the zero
// recurrent state.
int reset_rec_slot(spec_ctx* c, int seq) {
  if (!c->lo.any_rec) return SPEC_OK;
  int32_t* h = c->h_kvlen() + c->lo.max_seqs + seq;  // staging word next to the cache lengths
  *h = -1;
  HIPCHK(c, hipMemcpyAsync(c->ws<int32_t>(c->lo.rec_slot) + seq, h, 4, hipMemcpyHostToDevice, c->st));
  return SPEC_OK;
}

// -------------------------------------------------------- forward sequence

// The down projection reads the SwiGLU output as fp16 rows and the O
// projection the attention output, where their one-pass kernels serve the
// rows: bf16 weights, at most 8 rows (k_mm1l, k_mm1); int4 weights, the LDS
// or register kernel (k_mmq, k_mmqr); O only after an attention (not
// recurrent) layer.
bool int4_onepass(int K, int nk, int R) {
  int nk_mmq = nk;
  const int route = int4_route(K, nk, R, EPI_RESID, &nk_mmq);
  return route == INT4_MMQ || route == INT4_MMQR;
}
bool down_reads_h16(const spec_ctx* c, int R) {
  const Layout& L = c->lo;
  if (L.fmt == FMT_INT4) return R <= 16 && int4_onepass(L.F, L.nk_d, R);
  return L.d_lds && R <= 8;
}
bool o_reads_o16(const spec_ctx* c, int l, int R) {
  const Layout& L = c->lo;
  if (L.rec[(size_t)l]) return false;
  if (L.fmt == FMT_INT4) return R <= 16 && int4_onepass(L.DQ, L.nk_o, R);
  return R <= 8 && R <= L.mm_o.rmax && L.mm_o.nw == 8 && L.mm_o.spw == 16 && L.mm_o.nbuf == 0;
}

GemmParams gemm_common(spec_ctx* c, const void* W, int N, int K, int nk, int R) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.W = W;
  if (c->lo.fmt == FMT_INT4) p.scales = (const uint16_t*)((const uint8_t*)W + packed_int4_frag_bytes(N, K));
  p.N = N;
  p.K = K;
  p.R = R;
  p.nslices = K / (nk * 32);
  p.part = c->ws<float>(c->lo.part);
  p.cnt = c->ws<unsigned>(c->lo.cnt);
  p.eps = c->d.rms_eps;
  p.inv_dim = 1.0f / (float)c->lo.H;
  return p;
}

// R <= the plan's rmax (<= 16): the one-pass GEMM; above 16 rows (bf16) the
// many-row GEMM where the shape fits it, on A prepared once (by k_prep, or
// by its producer); otherwise split-K.
// ready: A already in the prepared layout, written by its producer (the
// SwiGLU epilogue, the attention merge) for this GEMM, or null.
hipError_t gemm_or_mm(const GemmParams& p0, const MmPlan& m, int nk, int epi, int fmt, int max_grid, void* af,
                      hipStream_t st, const void* ready = nullptr) {
  if (m.nw && p0.R <= m.rmax && p0.R <= 16) return launch_mm(p0, m.nw, m.spw, m.ct, m.nbuf, m.gp, max_grid, epi, st);
  if (fmt == FMT_INT4) {
    int nk_mmq = nk;
    const int route = int4_route(p0.K, nk, p0.R, epi, &nk_mmq);
    if (route == INT4_MMQ) return launch_mmq(p0, nk_mmq, epi, max_grid, st);
    if (route == INT4_MMQR) return launch_mmqr(p0, epi, max_grid, st);
  }
  // bf16 above 16 rows: the many-row GEMM on prepared A (its producer's, or k_prep's)
  const int ns_big = fmt == FMT_BF16 && p0.R > 16 && (ready || af) ? big_slices(p0.N, p0.K, epi) : 0;
  if (ns_big) {
    GemmParams p = p0;
    if (ready) {
      p.Af = ready;
    } else {
      const hipError_t e = launch_prep_a(p0, af, st);
      if (e != hipSuccess) return e;
      p.Af = af;
    }
    return launch_gemm_big(p, ns_big, SPECV_BIG_CT, epi, st);
  }
  return launch_gemm(p0, nk, epi, fmt, st);
}

// Per-op event hook for spec_profile_ops (null in the normal path).
struct OpTimer {
  std::vector<hipEvent_t>* ev;
  std::vector<int>* ops;
};

int mark(spec_ctx* c, OpTimer* t, int op) {
  if (!t) return SPEC_OK;
  hipEvent_t e;
  HIPCHK(c, hipEventCreate(&e));
  t->ev->push_back(e);
  t->ops->push_back(op);
  HIPCHK(c, hipEventRecord(e, c->st));
  return SPEC_OK;
}

#define STEP(call)                 \
  do {                             \
    int rc_ = (call);              \
    if (rc_ != SPEC_OK) return rc_; \
  } while (0)

// Launch one kernel of the forward: op class `op` of layer `l` (embed and LM
// ignore l) for n_seq sequences of S rows.
int launch_op(spec_ctx* c, int op, int l, int n_seq, int S) {
  const Layout& L = c->lo;
  const int R = n_seq * S;
  const StepDev* sd = c->ws<StepDev>(L.step);
  const int32_t* tokens = (const int32_t*)(sd + 1);
  const int32_t* seq_ids = tokens + L.max_rows;
  hipStream_t st = c->st;
  if (op == SPEC_OP_EMBED) {
    EmbedParams ep;
    ep.emb = (const uint16_t*)(c->W + L.emb);
    ep.tokens = tokens;
    ep.x = c->ws<float>(L.x);
    ep.ss = c->ws<float>(L.ss);
    ep.H = L.H;
    ep.seq_ids = seq_ids;
    ep.kv_len = c->ws<int32_t>(L.kv_len);
    ep.bt = c->ws<int32_t>(L.bt);
    ep.bt_stride = L.bt_stride;
    ep.S = S;
    ep.rowinfo = c->ws<int32_t>(L.rowinfo);
    ep.slotbt = c->ws<int32_t>(L.slotbt);
    HIPCHK(c, launch_embed(ep, R, st));
    return SPEC_OK;
  }
  if (op == SPEC_OP_LM) {
    GemmParams gl = gemm_common(c, c->W + L.wlm, L.V, L.H, L.nk_lm, R);
    gl.A = c->ws<float>(L.x);
    gl.lda = L.H;
    gl.ss = c->ws<float>(L.ss);
    gl.ss_n = L.H / 16;
    gl.gain = (const float*)(c->W + L.g_final);
    gl.argkey = c->ws<unsigned long long>(L.argkey);
    gl.lm_cnt = c->ws<unsigned>(L.lm_cnt);
    gl.status = c->ws<int32_t>(L.status);
    gl.logits = (c->d.flags & SPEC_FLAG_KEEP_LOGITS) ? c->ws<float>(L.logits) : nullptr;
    gl.tokens = tokens;
    gl.kd = seq_ids + L.max_rows;
    gl.mode = &sd->mode;
    gl.step = sd;
    gl.rowinfo = c->ws<int32_t>(L.rowinfo);
    gl.rec_slot = L.any_rec ? c->ws<int32_t>(L.rec_slot) : nullptr;
    gl.result = c->ws<int32_t>(L.result);
    gl.kv_len_w = c->ws<int32_t>(L.kv_len);
    gl.seq_ids = seq_ids;
    gl.S = S;
    gl.n_seq = n_seq;
    HIPCHK(c, gemm_or_mm(gl, L.mm_lm, L.nk_lm, EPI_LM, L.fmt, c->mm_grid, c->af(), st));
    return SPEC_OK;
  }
  const LayerOff& lw = L.lay[(size_t)l];
  switch (op) {
    case SPEC_OP_QKV: {  // QKV + RoPE + KV write
      GemmParams g = gemm_common(c, c->W + lw.wqkv, L.Nqkv, L.H, L.nk_qkv, R);
      g.A = c->ws<float>(L.x);
      g.lda = L.H;
      g.ss = c->ws<float>(L.ss);
      g.ss_n = L.H / 16;
      g.gain = (const float*)(c->W + lw.g_attn);
      g.q = c->ws<float>(L.q);
      g.q16 = L.rec[(size_t)l] ? nullptr : c->ws<_Float16>(L.q16);  // attention layers: fp16 queries
      g.kpool = c->kpool(l);
      g.vpool = c->vpool(l);
      g.bt = c->ws<int32_t>(L.bt);
      g.bt_stride = L.bt_stride;
      g.kv_len = c->ws<int32_t>(L.kv_len);
      g.seq_ids = seq_ids;
      g.S = S;
      g.n_q = L.nq;
      g.n_kv = L.nkv;
      g.hd = L.hd;
      g.rope = c->ws<float>(L.rope);
      g.rowinfo = c->ws<int32_t>(L.rowinfo);
      g.ring_nb = L.local[(size_t)l] ? L.ring_nb : 0;
      g.ring_w = L.local[(size_t)l] ? L.ring_w : 0;
      g.rec_kv = L.rec[(size_t)l] ? c->ws<float>(L.rec_kv) : nullptr;
      HIPCHK(c, gemm_or_mm(g, L.mm_qkv, L.nk_qkv, EPI_QKV, L.fmt, c->mm_grid, c->af(), st));
      return SPEC_OK;
    }
    case SPEC_OP_ATTN: {
      if (L.rec[(size_t)l]) {
        RecParams rp;
        rp.q = c->ws<float>(L.q);
        rp.kv = c->ws<float>(L.rec_kv);
        rp.snap = (float*)(c->KV + L.kv_off[(size_t)l]);
        rp.slot = c->ws<int32_t>(L.rec_slot);
        rp.seq_ids = seq_ids;
        rp.out = c->ws<float>(L.o);
        rp.af_out = c->af_next(L.H, L.DQ, R);
        rp.S = S;
        rp.n_seq = n_seq;
        rp.n_q = L.nq;
        rp.n_kv = L.nkv;
        rp.beta = c->d.rec_beta;
        HIPCHK(c, launch_recur(rp, L.hd, st));
        return SPEC_OK;
      }
      AttnParams a;
      a.q = c->ws<_Float16>(L.q16);
      a.kpool = c->kpool(l);
      a.vpool = c->vpool(l);
      a.rowinfo = c->ws<int32_t>(L.rowinfo);
      a.slotbt = c->ws<int32_t>(L.slotbt);
      a.bt_stride = L.bt_stride;
      a.S = S;
      a.n_seq = n_seq;
      a.n_q = L.nq;
      a.n_kv = L.nkv;
      a.scale = (float)(1.0 / sqrt((double)L.hd));
      a.max_splits = L.max_splits;
      a.part = c->ws<float>(L.apart);
      a.cnt = c->ws<unsigned>(L.attn_cnt);
      a.out = c->ws<float>(L.o);
      a.out16 = o_reads_o16(c, l, R) ? c->ws<_Float16>(L.o16) : nullptr;
      a.af_out = c->af_next(L.H, L.DQ, R);
      a.n_qt = (S * L.G + 15) / 16;
      const bool loc = L.local[(size_t)l] != 0;
      a.tpw = std::min(loc ? c->attn_tpw_l : c->attn_tpw, a.n_qt);
      a.fuse = loc ? c->attn_fuse_l : c->attn_fuse;
      a.win = loc ? L.win : 0;
      a.ring_nb = loc ? L.ring_nb : 0;
      a.ring_w = loc ? L.ring_w : 0;
      a.grid_splits = loc ? L.win_splits : L.max_splits;
      a.seq_ids = seq_ids;
      HIPCHK(c, launch_attn(a, L.hd, st));
      return SPEC_OK;
    }
    case SPEC_OP_O: {
      GemmParams go = gemm_common(c, c->W + lw.wo, L.H, L.DQ, L.nk_o, R);
      go.A = c->ws<float>(L.o);
      go.lda = L.DQ;
      go.x = c->ws<float>(L.x);
      go.ss_out = c->ws<float>(L.ss);
      if (o_reads_o16(c, l, R)) go.A16 = c->ws<_Float16>(L.o16);
      // up to four rows of the eight-part plan: the same K parts with A staged in LDS
      if (SPECV_O_LDS && L.fmt == FMT_BF16 && R <= 4 && L.mm_o.nw == 8 && L.mm_o.spw == 16 && L.mm_o.nbuf == 0 &&
          L.mm_o.gp == 1 && R <= L.mm_o.rmax) {
        HIPCHK(c, launch_mm1l(go, 8, 16, 4, st));
        return SPEC_OK;
      }
      HIPCHK(c, gemm_or_mm(go, L.mm_o, L.nk_o, EPI_RESID, L.fmt, c->mm_grid, c->af(), st, c->af_next(L.H, L.DQ, R)));
      return SPEC_OK;
    }
    case SPEC_OP_GATEUP: {
      GemmParams gu = gemm_common(c, c->W + lw.wgu, L.Ngu, L.H, L.nk_gu, R);
      gu.A = c->ws<float>(L.x);
      gu.lda = L.H;
      gu.ss = c->ws<float>(L.ss);
      gu.ss_n = L.H / 16;
      gu.gain = (const float*)(c->W + lw.g_ffn);
      gu.h = c->ws<float>(L.h);
      gu.h16 = down_reads_h16(c, R) ? c->ws<_Float16>(L.h16) : nullptr;
      gu.af_out = c->af_next(L.H, L.F, R);
      HIPCHK(c, gemm_or_mm(gu, L.mm_gu, L.nk_gu, EPI_SWIGLU, L.fmt, c->mm_grid, c->af(), st));
      return SPEC_OK;
    }
    case SPEC_OP_DOWN: {
      GemmParams gd = gemm_common(c, c->W + lw.wd, L.H, L.F, L.nk_d, R);
      gd.A = c->ws<float>(L.h);
      gd.lda = L.F;
      gd.x = c->ws<float>(L.x);
      gd.ss_out = c->ws<float>(L.ss);
      if (down_reads_h16(c, R)) gd.A16 = c->ws<_Float16>(L.h16);
      if (L.d_lds && R <= 8) HIPCHK(c, launch_mm1l(gd, 16, 19, 8, st));
      else if (L.d_lds && R <= SPECV_DOWN_MM1_ROWS)
        HIPCHK(c, launch_mm(gd, 16, 19, 4, 0, 1, c->mm_grid, EPI_RESID, st));
      else HIPCHK(c, gemm_or_mm(gd, L.mm_d, L.nk_d, EPI_RESID, L.fmt, c->mm_grid, c->af(), st, c->af_next(L.H, L.F, R)));
      return SPEC_OK;
    }
  }
  return set_err(c, SPEC_EINVAL, "unknown op class");
}

int enqueue_forward(spec_ctx* c, int n_seq, int S, OpTimer* tm) {
  STEP(mark(c, tm, SPEC_OP_EMBED));
  STEP(launch_op(c, SPEC_OP_EMBED, 0, n_seq, S));
  for (int l = 0; l < c->lo.L; ++l) {
    for (int op : {SPEC_OP_QKV, SPEC_OP_ATTN, SPEC_OP_O, SPEC_OP_GATEUP, SPEC_OP_DOWN}) {
      STEP(mark(c, tm, op));
      STEP(launch_op(c, op, l, n_seq, S));
    }
  }
  STEP(mark(c, tm, SPEC_OP_LM));
  STEP(launch_op(c, SPEC_OP_LM, 0, n_seq, S));
  STEP(mark(c, tm, -1));
  return SPEC_OK;
}

int get_graph(spec_ctx* c, int n_seq, int S, hipGraphExec_t* out) {
  auto key = std::make_pair(n_seq, S | (c->attn_fuse << 16) | (c->attn_fuse_l << 17) | ((c->attn_tpw & 31) << 18) |
                                       ((c->attn_tpw_l & 31) << 23));
  auto it = c->graphs.find(key);
  if (it != c->graphs.end()) {
    *out = it->second;
    return SPEC_OK;
  }
  HIPCHK(c, hipStreamBeginCapture(c->st, hipStreamCaptureModeThreadLocal));
  const int rc = enqueue_forward(c, n_seq, S, nullptr);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(c->st, &g);
  if (rc != SPEC_OK) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return set_err(c, SPEC_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  hipGraphExec_t ge = nullptr;
  const hipError_t e2 = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e2 != hipSuccess) return set_err(c, SPEC_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e2));
  c->graphs[key] = ge;
  c->stats.graphs++;
  *out = ge;
  return SPEC_OK;
}

// Stage the step block (mode, shape, tokens, sequence ids, drafts per
// sequence) and copy it; pick the attention variant of the step from the
// host's cache lengths.  kd: drafts per sequence, or null for S - 1 each.
int upload_step(spec_ctx* c, int mode, int n_seq, int S, const int32_t* tokens, const int32_t* seq_ids,
                const int32_t* kd = nullptr) {
  const Layout& L = c->lo;
  int longest = 0;
  for (int b = 0; b < n_seq; ++b) longest = std::max(longest, c->len[(size_t)seq_ids[b]] + S);
  // Enough (sequence, kv head, split) workgroups to fill the chip, and more
  // than SPECV_ATTN_TPW1_WGS of them with one query tile each: each takes its
  // query tiles on K and V loaded once, all of them when they are at most two
  // (one pass of the two-tile kernel), else two per workgroup (three or four
  // tiles in one workgroup took two passes each: 35.2 against 33.8 us at five
  // rows of the 32B-class heads over 8192 tokens); else one tile each (the
  // tiles of a long span side by side).
  const int splits = (longest + 255) / 256, n_qt = (S * L.G + 15) / 16;
  auto tiles_per_wg = [&](int sp) {
    const size_t wg = (size_t)n_seq * L.nkv * sp;
    return (wg >= 256 && wg * n_qt > (size_t)SPECV_ATTN_TPW1_WGS) ? (n_qt >= 3 ? 2 : 16) : 1;
  };
  c->attn_tpw = tiles_per_wg(splits);
  // The last split merges its tile group itself when that is short work: few
  // splits per column and at most two tiles; else the merge kernel spreads
  // the columns over the chip.
  c->attn_fuse = (splits <= std::min(SPECV_ATTN_FUSE_SPLITS, attn_fuse_splits(L.hd)) &&
                  std::min(c->attn_tpw, n_qt) <= 2) ? 1 : 0;
  // sliding-window layers: at most the splits a window touches
  const int splits_l = L.win > 0 ? std::min(splits, L.win_splits) : splits;
  c->attn_tpw_l = tiles_per_wg(splits_l);
  c->attn_fuse_l = (splits_l <= std::min(SPECV_ATTN_FUSE_SPLITS, attn_fuse_splits(L.hd)) &&
                    std::min(c->attn_tpw_l, n_qt) <= 2) ? 1 : 0;
  StepDev* sd = (StepDev*)c->h_step();
  sd->mode = mode;
  sd->n_seq = n_seq;
  sd->span = S;
  sd->pad = 0;
  sd->temp = c->temp;
  sd->seed_lo = (uint32_t)c->seed;
  sd->seed_hi = (uint32_t)(c->seed >> 32);
  sd->pad2 = 0;
  int32_t* tk = (int32_t*)(sd + 1);
  memcpy(tk, tokens, sizeof(int32_t) * (size_t)n_seq * S);
  memcpy(tk + L.max_rows, seq_ids, sizeof(int32_t) * (size_t)n_seq);
  int32_t* kdev = tk + 2 * L.max_rows;
  for (int b = 0; b < n_seq; ++b) kdev[b] = kd ? kd[b] : S - 1;
  const size_t bytes = sizeof(StepDev) + (size_t)L.max_rows * 8 + (size_t)n_seq * 4;
  // tokens of the whole row range and the used sequence ids, in one copy
  HIPCHK(c, hipMemcpyAsync(c->ws<uint8_t>(L.step), c->h_step(), bytes, hipMemcpyHostToDevice, c->st));
  return SPEC_OK;
}

int launch_forward(spec_ctx* c, int n_seq, int S) {
  if (c->d.flags & SPEC_FLAG_NO_GRAPH) return enqueue_forward(c, n_seq, S, nullptr);
  hipGraphExec_t ge;
  STEP(get_graph(c, n_seq, S, &ge));
  HIPCHK(c, hipGraphLaunch(ge, c->st));
  return SPEC_OK;
}

// One forward and its result copy; synchronous.  Verify forwards are timed
// with the context's two events (forward launch to accept done) into the
// per-span totals of spec_get_stats.
int run_forward(spec_ctx* c, int mode, int n_seq, int S, const int32_t* tokens, const int32_t* seq_ids,
                const int32_t* kd = nullptr) {
  STEP(upload_step(c, mode, n_seq, S, tokens, seq_ids, kd));
  const bool timed = mode == MODE_VERIFY && c->ev0 && c->ev1;
  if (timed) HIPCHK(c, hipEventRecord(c->ev0, c->st));
  STEP(launch_forward(c, n_seq, S));
  if (timed) HIPCHK(c, hipEventRecord(c->ev1, c->st));
  HIPCHK(c, hipMemcpyAsync(c->h_result(), c->ws<int32_t>(c->lo.result), (size_t)(1 + n_seq * (S + 1)) * 4,
                           hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  if (timed) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, c->ev0, c->ev1) == hipSuccess) c->stats.forward_ms_by_span[S] += ms;
  }
  c->stats.forwards++;
  c->last_rows = n_seq * S;
  if (c->h_result()[0] & 1) return set_err(c, SPEC_ENAN, "a logit row held NaN");
  return SPEC_OK;
}

int check_ready(spec_ctx* c) {
  if (!all_loaded(c)) return set_err(c, SPEC_ESTATE, "weights not fully loaded");
  return SPEC_OK;
}

int check_tokens(spec_ctx* c, const int32_t* t, int n) {
  for (int i = 0; i < n; ++i)
    if (t[i] < 0 || t[i] >= c->lo.V) return set_err(c, SPEC_EINVAL, "token outside [0, vocab)");
  return SPEC_OK;
}

int check_seq(spec_ctx* c, int seq) {
  if (seq < 0 || seq >= c->lo.max_seqs) return set_err(c, SPEC_EINVAL, "sequence id out of range");
  return SPEC_OK;
}

}  // namespace

// =================================================================== ABI

extern "C" {

int spec_query_buffers(const spec_model_desc* desc, spec_buffer_sizes* out) {
  if (!desc || !out) return SPEC_EINVAL;
  Layout L;
  if (!build_layout(*desc, L, g_create_error)) return SPEC_EINVAL;
  out->weights_bytes = L.weights_bytes;
  out->kv_bytes = L.kv_bytes;
  out->workspace_bytes = L.workspace_bytes;
  out->host_bytes = L.host_bytes;
  return SPEC_OK;
}

const char* spec_last_error(const spec_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_error.c_str(); }

}  // extern "C"

namespace {

// no_alloc: the context of spec_create_static -- eager launches (no graph
// objects) and no timing events, so that nothing beyond host memory is
// allocated.
int create_impl(const spec_model_desc* desc, const spec_device_buffers* b, void* hip_stream, spec_ctx** out,
                bool no_alloc) {
  if (!desc || !b || !out) {
    g_create_error = "null argument";
    return SPEC_EINVAL;
  }
  *out = nullptr;
  if (desc->flags & ~(SPEC_FLAG_KEEP_LOGITS | SPEC_FLAG_NO_GRAPH)) {
    g_create_error = "unknown flag bits";
    return SPEC_EINVAL;
  }
  spec_ctx* c = new (std::nothrow) spec_ctx;
  if (!c) {
    g_create_error = "out of host memory";
    return SPEC_ECAPACITY;
  }
  c->d = *desc;
  if (no_alloc) c->d.flags |= SPEC_FLAG_NO_GRAPH;
  if (!build_layout(*desc, c->lo, g_create_error)) {
    delete c;
    return SPEC_EINVAL;
  }
  const Layout& L = c->lo;
  if (!b->weights || !b->kv || !b->workspace || !b->host || b->weights_bytes < L.weights_bytes ||
      b->kv_bytes < L.kv_bytes || b->workspace_bytes < L.workspace_bytes || b->host_bytes < L.host_bytes) {
    g_create_error = "a buffer is missing or smaller than spec_query_buffers reports";
    delete c;
    return SPEC_ECAPACITY;
  }
  if (((uintptr_t)b->weights | (uintptr_t)b->kv | (uintptr_t)b->workspace) & (kAlign - 1)) {
    g_create_error = "device buffers must be 256-byte aligned";
    delete c;
    return SPEC_EINVAL;
  }
  if (!hip_stream) {
    g_create_error = "a non-NULL HIP stream is required";
    delete c;
    return SPEC_EINVAL;
  }
  c->st = (hipStream_t)hip_stream;
  c->W = (uint8_t*)b->weights;
  c->KV = (uint8_t*)b->kv;
  c->WS = (uint8_t*)b->workspace;
  c->HB = (uint8_t*)b->host;
  c->len.assign((size_t)L.max_seqs, 0);
  c->nblk.assign((size_t)L.max_seqs, 0);
  c->live.assign((size_t)L.max_seqs, 0);
  for (int i = L.n_blocks - 1; i >= 0; --i) c->free_blocks.push_back(i);
  c->loaded.assign((size_t)n_slots(c), 0u);
  memset(&c->stats, 0, sizeof(c->stats));
  memset(c->HB, 0, L.host_bytes);

  // Zero the KV pool (masked keys multiply exact zeros, never stale NaN) and
  // the workspace (counters, maxima and cache lengths start at zero).
  hipError_t e = launch_fill_u32(c->KV, 0u, L.kv_bytes / 4, c->st);
  if (e == hipSuccess) e = launch_fill_u32(c->WS, 0u, L.workspace_bytes / 4, c->st);
  // RoPE table: angle pos * theta^(-2j/hd) in fp64, stored as fp32 (cos, sin).
  std::vector<float> rope((size_t)L.max_ctx * (L.hd / 2) * 2);
  for (int pos = 0; pos < L.max_ctx; ++pos)
    for (int j = 0; j < L.hd / 2; ++j) {
      const double ang = (double)pos * pow(desc->rope_theta, -2.0 * j / (double)L.hd);
      rope[((size_t)pos * (L.hd / 2) + j) * 2] = (float)cos(ang);
      rope[((size_t)pos * (L.hd / 2) + j) * 2 + 1] = (float)sin(ang);
    }
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->WS + L.rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice, c->st);
  if (e == hipSuccess) e = hipStreamSynchronize(c->st);
  if (e != hipSuccess) {
    g_create_error = std::string("initialising device buffers: ") + hipGetErrorString(e);
    delete c;
    return SPEC_EHIP;
  }
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      g_create_error = "cannot read the device's compute unit count";
      delete c;
      return SPEC_EHIP;
    }
    c->mm_grid = cus * SPECV_MM_WG_PER_CU;  // one resident workgroup per CU walks the blocks
  }
  if (!no_alloc && (hipEventCreate(&c->ev0) != hipSuccess || hipEventCreate(&c->ev1) != hipSuccess)) {
    g_create_error = "cannot create the forward timing events";
    if (c->ev0) (void)hipEventDestroy(c->ev0);
    delete c;
    return SPEC_EHIP;
  }
  *out = c;
  return SPEC_OK;
}

}  // namespace

// Scratch of the allocation-free entry point: the workspace of the one live
// static context per GPU, in the library's own device memory (each GPU the
// library runs on holds its copy until the process ends).  Host code never
// uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, at the device's first
// spec_create_static.
static __device__ __align__(256) uint8_t scratch[SPEC_STATIC_SCRATCH_BYTES];

namespace {

struct StaticSlot {
  void* ptr = nullptr;      // this device's copy of `scratch`
  spec_ctx* owner = nullptr;  // the live static context on this device, if any
};
std::mutex g_static_mu;
std::vector<StaticSlot> g_static;  // by device ordinal

}  // namespace

extern "C" {

int spec_create(const spec_model_desc* desc, const spec_device_buffers* b, void* hip_stream, spec_ctx** out) {
  return create_impl(desc, b, hip_stream, out, false);
}

int spec_create_static(const spec_model_desc* desc, const spec_device_buffers* bufs, void* hip_stream,
                       spec_ctx** out) {
  if (!desc || !bufs || !out) {
    g_create_error = "null argument";
    return SPEC_EINVAL;
  }
  *out = nullptr;
  if (bufs->workspace || bufs->workspace_bytes) {
    g_create_error = "spec_create_static takes no workspace: the library's static scratch is the workspace";
    return SPEC_EINVAL;
  }
  Layout L;
  if (!build_layout(*desc, L, g_create_error)) return SPEC_EINVAL;
  if (L.workspace_bytes > (size_t)SPEC_STATIC_SCRATCH_BYTES) {
    g_create_error = "this description needs " + std::to_string(L.workspace_bytes) +
                     " bytes of workspace, more than the static scratch of " +
                     std::to_string((size_t)SPEC_STATIC_SCRATCH_BYTES) + " bytes";
    return SPEC_ECAPACITY;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_create_error = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return SPEC_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_static_mu);
  if ((size_t)dev >= g_static.size()) g_static.resize((size_t)dev + 1);
  StaticSlot& slot = g_static[(size_t)dev];
  if (!slot.ptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_create_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return SPEC_EHIP;
    }
    slot.ptr = ptr;
  }
  if (slot.owner) {
    g_create_error = "a static context already lives on this device (they share its scratch)";
    return SPEC_ESTATE;
  }
  spec_device_buffers b = *bufs;
  b.workspace = slot.ptr;
  b.workspace_bytes = (size_t)SPEC_STATIC_SCRATCH_BYTES;
  const int rc = create_impl(desc, &b, hip_stream, out, true);
  if (rc != SPEC_OK) return rc;
  (*out)->static_dev = dev;
  slot.owner = *out;
  return SPEC_OK;
}

int spec_destroy(spec_ctx* c) {
  if (!c) return SPEC_EINVAL;
  if (c->static_dev >= 0) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    g_static[(size_t)c->static_dev].owner = nullptr;
  }
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  if (c->ev0) (void)hipEventDestroy(c->ev0);
  if (c->ev1) (void)hipEventDestroy(c->ev1);
  delete c;
  return SPEC_OK;
}

// Pack one canonical matrix (rows x cols, source row s -> fused row map(s))
// into the fused matrix at dst of the context's weight format.
static hipError_t pack_matrix(spec_ctx* c, const void* src, const void* scales, int rows, int cols, uint8_t* dst,
                              int fused_rows, int kind, int row0, int hd) {
  if (c->lo.fmt == FMT_INT4)
    return launch_pack_int4((const uint8_t*)src, (const uint16_t*)scales, rows, cols, dst,
                            (uint16_t*)(dst + packed_int4_frag_bytes(fused_rows, cols)), kind, row0, hd, c->st);
  return launch_pack_bf16((const uint16_t*)src, rows, cols, dst, kind, row0, hd, c->ws<uint32_t>(c->lo.packflag),
                          c->st);
}

int spec_load_matrix(spec_ctx* c, int layer, int which, const void* src, const void* scales) {
  if (!c || !src) return c ? set_err(c, SPEC_EINVAL, "null source") : SPEC_EINVAL;
  if (c->lo.fmt == FMT_INT4 && which != SPEC_MAT_EMB && !scales)
    return set_err(c, SPEC_EINVAL, "int4 matrices need their scales");
  const Layout& L = c->lo;
  const bool global = (which == SPEC_MAT_EMB || which == SPEC_MAT_LM);
  if (which < 0 || which > SPEC_MAT_LM) return set_err(c, SPEC_EINVAL, "unknown matrix id");
  if (!global && (layer < 0 || layer >= L.L)) return set_err(c, SPEC_EINVAL, "layer out of range");
  hipError_t e = hipSuccess;
  int slot_id;
  if (which == SPEC_MAT_EMB) {
    e = hipMemcpyAsync(c->W + L.emb, src, (size_t)L.V * L.H * 2, hipMemcpyDeviceToDevice, c->st);
    slot_id = L.L * 9 + 0;
  } else if (which == SPEC_MAT_LM) {
    e = pack_matrix(c, src, scales, L.V, L.H, c->W + L.wlm, L.V, 0, 0, 0);
    slot_id = L.L * 9 + 1;
  } else {
    const LayerOff& lw = L.lay[(size_t)layer];
    switch (which) {
      case SPEC_MAT_Q: e = pack_matrix(c, src, scales, L.DQ, L.H, c->W + lw.wqkv, L.Nqkv, 1, 0, L.hd); break;
      case SPEC_MAT_K: e = pack_matrix(c, src, scales, L.DK, L.H, c->W + lw.wqkv, L.Nqkv, 1, L.DQ, L.hd); break;
      case SPEC_MAT_V: e = pack_matrix(c, src, scales, L.DK, L.H, c->W + lw.wqkv, L.Nqkv, 0, L.DQ + L.DK, 0); break;
      case SPEC_MAT_O: e = pack_matrix(c, src, scales, L.H, L.DQ, c->W + lw.wo, L.H, 0, 0, 0); break;
      case SPEC_MAT_GATE: e = pack_matrix(c, src, scales, L.F, L.H, c->W + lw.wgu, L.Ngu, 2, 0, 0); break;
      case SPEC_MAT_UP: e = pack_matrix(c, src, scales, L.F, L.H, c->W + lw.wgu, L.Ngu, 2, 1, 0); break;
      case SPEC_MAT_DOWN: e = pack_matrix(c, src, scales, L.H, L.F, c->W + lw.wd, L.H, 0, 0, 0); break;
    }
    slot_id = slot(c, layer, which);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(c->st);
  if (e != hipSuccess) return set_err(c, SPEC_EHIP, std::string("weight packing: ") + hipGetErrorString(e));
  if (L.fmt == FMT_BF16 && which != SPEC_MAT_EMB) {
    // the GEMMs take fp16 copies of bf16 weights: refuse a matrix with a
    // value beyond the fp16 range
    uint32_t over = 0;
    e = hipMemcpy(&over, c->ws<uint32_t>(L.packflag), 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return set_err(c, SPEC_EHIP, std::string("weight packing: ") + hipGetErrorString(e));
    if (over) {
      c->loaded[(size_t)slot_id] = 0u;
      e = launch_fill_u32(c->ws<uint32_t>(L.packflag), 0u, 1, c->st);
      if (e == hipSuccess) e = hipStreamSynchronize(c->st);
      return set_err(c, SPEC_EINVAL, "a bf16 weight is beyond the fp16 range (|w| > 65504)");
    }
  }
  c->loaded[(size_t)slot_id] = 1u;
  return SPEC_OK;
}

int spec_load_norm(spec_ctx* c, int layer, int which, const float* src) {
  if (!c || !src) return c ? set_err(c, SPEC_EINVAL, "null source") : SPEC_EINVAL;
  const Layout& L = c->lo;
  size_t off;
  int slot_id;
  if (which == SPEC_NORM_FINAL) {
    off = L.g_final;
    slot_id = L.L * 9 + 2;
  } else {
    if (layer < 0 || layer >= L.L) return set_err(c, SPEC_EINVAL, "layer out of range");
    if (which == SPEC_NORM_ATTN) off = L.lay[(size_t)layer].g_attn;
    else if (which == SPEC_NORM_FFN) off = L.lay[(size_t)layer].g_ffn;
    else return set_err(c, SPEC_EINVAL, "unknown norm id");
    slot_id = slot(c, layer, 7 + which);
  }
  HIPCHK(c, hipMemcpyAsync(c->W + off, src, (size_t)L.H * 4, hipMemcpyDeviceToDevice, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  c->loaded[(size_t)slot_id] = 1u;
  return SPEC_OK;
}

int spec_prefill_seq(spec_ctx* c, int seq, const int32_t* tokens, int n, int32_t* next_token) {
  if (!c) return SPEC_EINVAL;
  if (!tokens || !next_token || n <= 0) return set_err(c, SPEC_EINVAL, "prefill needs n >= 1 tokens");
  STEP(check_seq(c, seq));
  STEP(check_ready(c));
  STEP(check_tokens(c, tokens, n));
  if (n > c->lo.max_ctx) return set_err(c, SPEC_ECAPACITY, "prompt longer than max_ctx");
  c->len[(size_t)seq] = 0;
  c->live[(size_t)seq] = 0;
  trim_blocks(c, seq, 0);
  STEP(upload_kv_len(c, seq));
  STEP(reset_rec_slot(c, seq));
  const int chunk = std::min(SPEC_MAX_SPAN, c->lo.max_rows);
  int g = -1;
  for (int off = 0; off < n; off += chunk) {
    const int S = std::min(chunk, n - off);
    bool dirty = false;
    int rc = ensure_blocks(c, seq, off + S, &dirty);
    if (rc == SPEC_OK && dirty) rc = upload_bt_row(c, seq);
    const int32_t sid = seq;
    if (rc == SPEC_OK) rc = run_forward(c, MODE_COMMIT_ALL, 1, S, tokens + off, &sid);
    if (rc != SPEC_OK) {
      // a failed chunk leaves the sequence empty (not half prefilled) on
      // both sides
      c->len[(size_t)seq] = 0;
      trim_blocks(c, seq, 0);
      (void)upload_kv_len(c, seq);
      (void)reset_rec_slot(c, seq);
      (void)hipStreamSynchronize(c->st);
      return rc;
    }
    c->len[(size_t)seq] += S;
    g = c->h_result()[1 + 1 + (S - 1)];
  }
  c->live[(size_t)seq] = 1;
  *next_token = g;
  return SPEC_OK;
}

int spec_prefill(spec_ctx* c, const int32_t* tokens, int n, int32_t* next_token) {
  return spec_prefill_seq(c, 0, tokens, n, next_token);
}

int spec_verify_batch_k(spec_ctx* c, int n_seq, const int32_t* seq_ids, const int32_t* spans, int K,
                        const int32_t* drafts, int32_t* argmax, int32_t* accept_len) {
  if (!c) return SPEC_EINVAL;
  if (!seq_ids || !spans || !argmax || !accept_len || n_seq <= 0)
    return set_err(c, SPEC_EINVAL, "null argument or n_seq < 1");
  const int S = K + 1;
  if (K < 0 || S > SPEC_MAX_SPAN) return set_err(c, SPEC_EINVAL, "K must be in [0, 15]");
  if (drafts)
    for (int b = 0; b < n_seq; ++b)
      if (drafts[b] < 0 || drafts[b] > K) return set_err(c, SPEC_EINVAL, "drafts per sequence must be in [0, K]");
  if (n_seq * S > c->lo.max_rows) return set_err(c, SPEC_EINVAL, "n_seq*(K+1) exceeds max_rows");
  STEP(check_ready(c));
  STEP(check_tokens(c, spans, n_seq * S));
  for (int b = 0; b < n_seq; ++b) {
    STEP(check_seq(c, seq_ids[b]));
    for (int j = 0; j < b; ++j)
      if (seq_ids[j] == seq_ids[b]) return set_err(c, SPEC_EINVAL, "duplicate sequence id");
    if (!c->live[(size_t)seq_ids[b]]) return set_err(c, SPEC_ESTATE, "verify before prefill");
    if (c->len[(size_t)seq_ids[b]] + S > c->lo.max_ctx)
      return set_err(c, SPEC_ECAPACITY, "cache length + span exceeds max_ctx");
  }
  for (int b = 0; b < n_seq; ++b) {
    const int seq = seq_ids[b];
    bool dirty = false;
    const int rc = ensure_blocks(c, seq, c->len[(size_t)seq] + S, &dirty);
    if (rc != SPEC_OK) {  // give back what this call took
      for (int j = 0; j <= b; ++j) trim_blocks(c, seq_ids[j], c->len[(size_t)seq_ids[j]]);
      return rc;
    }
    if (dirty) STEP(upload_bt_row(c, seq));
  }
  const int frc = run_forward(c, MODE_VERIFY, n_seq, S, spans, seq_ids, drafts);
  if (frc != SPEC_OK) {
    // The accept stage does not advance a cache on a NaN row; after any
    // failure the device lengths are set back to the host's (unchanged)
    // mirror and the blocks this call took are returned, so host and device
    // agree on every sequence's length and blocks.
    for (int b = 0; b < n_seq; ++b) {
      trim_blocks(c, seq_ids[b], c->len[(size_t)seq_ids[b]]);
      (void)upload_kv_len(c, seq_ids[b]);
    }
    (void)hipStreamSynchronize(c->st);
    return frc;
  }
  const int32_t* res = c->h_result() + 1;
  for (int b = 0; b < n_seq; ++b) {
    const int m = res[b * (S + 1)];
    accept_len[b] = m;
    memcpy(argmax + (size_t)b * S, res + b * (S + 1) + 1, sizeof(int32_t) * (size_t)S);
    const int seq = seq_ids[b];
    c->len[(size_t)seq] += m + 1;
    trim_blocks(c, seq, c->len[(size_t)seq]);
    c->stats.drafted += drafts ? drafts[b] : K;
    c->stats.accepted += m;
  }
  c->stats.verify_calls++;
  c->stats.forwards_by_span[S]++;
  return SPEC_OK;
}

int spec_verify_batch(spec_ctx* c, int n_seq, const int32_t* seq_ids, const int32_t* spans, int K,
                      int32_t* argmax, int32_t* accept_len) {
  return spec_verify_batch_k(c, n_seq, seq_ids, spans, K, nullptr, argmax, accept_len);
}

int spec_verify(spec_ctx* c, const int32_t* span, int K, int32_t* argmax, int32_t* accept_len) {
  const int32_t sid = 0;
  return spec_verify_batch(c, 1, &sid, span, K, argmax, accept_len);
}

int spec_rewind_seq(spec_ctx* c, int seq, int len) {
  if (!c) return SPEC_EINVAL;
  STEP(check_seq(c, seq));
  if (len < 0 || len > c->len[(size_t)seq]) return set_err(c, SPEC_ESTATE, "rewind length outside [0, cache length]");
  if (c->lo.any_rec && len != c->len[(size_t)seq] && len != 0)
    return set_err(c, SPEC_ESTATE, "a model with recurrent layers rewinds only to 0 (its state has no history)");
  c->len[(size_t)seq] = len;
  trim_blocks(c, seq, len);
  STEP(upload_kv_len(c, seq));
  if (len == 0) STEP(reset_rec_slot(c, seq));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return SPEC_OK;
}

int spec_rewind(spec_ctx* c, int len) { return spec_rewind_seq(c, 0, len); }

int spec_cache_len_seq(spec_ctx* c, int seq, int* len) {
  if (!c || !len) return SPEC_EINVAL;
  STEP(check_seq(c, seq));
  *len = c->len[(size_t)seq];
  return SPEC_OK;
}

int spec_cache_len(spec_ctx* c, int* len) { return spec_cache_len_seq(c, 0, len); }

int spec_release_seq(spec_ctx* c, int seq) {
  if (!c) return SPEC_EINVAL;
  STEP(check_seq(c, seq));
  c->len[(size_t)seq] = 0;
  c->live[(size_t)seq] = 0;
  trim_blocks(c, seq, 0);
  STEP(upload_kv_len(c, seq));
  STEP(reset_rec_slot(c, seq));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return SPEC_OK;
}

int spec_debug_logits(spec_ctx* c, float* host_out, int rows) {
  if (!c || !host_out) return SPEC_EINVAL;
  if (!(c->d.flags & SPEC_FLAG_KEEP_LOGITS)) return set_err(c, SPEC_ESTATE, "context built without KEEP_LOGITS");
  if (rows < 0 || rows > c->last_rows) return set_err(c, SPEC_EINVAL, "rows beyond the last forward");
  HIPCHK(c, hipMemcpyAsync(host_out, c->WS + c->lo.logits, (size_t)rows * c->lo.V * 4, hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return SPEC_OK;
}

int spec_set_sampling(spec_ctx* c, float temperature, uint64_t seed) {
  if (!c) return SPEC_EINVAL;
  if (!(temperature >= 0.0f) || temperature > 1e30f) return set_err(c, SPEC_EINVAL, "temperature must be >= 0 and finite");
  c->temp = temperature;
  c->seed = seed;
  return SPEC_OK;
}

int spec_get_stats(spec_ctx* c, spec_stats* out) {
  if (!c || !out) return SPEC_EINVAL;
  *out = c->stats;
  return SPEC_OK;
}

int spec_time_verify(spec_ctx* c, int S, int iters, const int32_t* spans, float* ms_out) {
  if (!c || !spans || !ms_out || iters <= 0) return c ? set_err(c, SPEC_EINVAL, "bad timing arguments") : SPEC_EINVAL;
  if (S < 1 || S > SPEC_MAX_SPAN || S > c->lo.max_rows) return set_err(c, SPEC_EINVAL, "S must be in [1, 16]");
  STEP(check_ready(c));
  STEP(check_tokens(c, spans, S * iters));
  if (!c->live[0]) return set_err(c, SPEC_ESTATE, "timing before prefill");
  if (c->len[0] + S > c->lo.max_ctx) return set_err(c, SPEC_ECAPACITY, "cache length + span exceeds max_ctx");
  bool dirty = false;
  STEP(ensure_blocks(c, 0, c->len[0] + S, &dirty));
  if (dirty) STEP(upload_bt_row(c, 0));
  hipEvent_t e0, e1;
  HIPCHK(c, hipEventCreate(&e0));
  HIPCHK(c, hipEventCreate(&e1));
  const int32_t sid = 0;
  int rc = SPEC_OK;
  for (int it = 0; it < iters && rc == SPEC_OK; ++it) {
    rc = upload_step(c, MODE_NO_COMMIT, 1, S, spans + (size_t)it * S, &sid);
    if (rc != SPEC_OK) break;
    hipError_t e = hipEventRecord(e0, c->st);
    if (e == hipSuccess) {
      rc = launch_forward(c, 1, S);
      if (rc != SPEC_OK) break;
      e = hipEventRecord(e1, c->st);
    }
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms_out[it], e0, e1);
    if (e != hipSuccess) rc = set_err(c, SPEC_EHIP, std::string("timing: ") + hipGetErrorString(e));
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  trim_blocks(c, 0, c->len[0]);
  c->last_rows = S;
  return rc;
}

int spec_profile_ops(spec_ctx* c, int S, int iters, const int32_t* spans, float* us_out, int32_t* launches_out) {
  if (!c || !spans || !us_out || !launches_out || iters <= 0)
    return c ? set_err(c, SPEC_EINVAL, "bad profiling arguments") : SPEC_EINVAL;
  if (S < 1 || S > SPEC_MAX_SPAN || S > c->lo.max_rows) return set_err(c, SPEC_EINVAL, "S must be in [1, 16]");
  STEP(check_ready(c));
  STEP(check_tokens(c, spans, S * iters));
  if (!c->live[0]) return set_err(c, SPEC_ESTATE, "profiling before prefill");
  if (c->len[0] + S > c->lo.max_ctx) return set_err(c, SPEC_ECAPACITY, "cache length + span exceeds max_ctx");
  bool dirty = false;
  STEP(ensure_blocks(c, 0, c->len[0] + S, &dirty));
  if (dirty) STEP(upload_bt_row(c, 0));
  double tot[SPEC_OP_COUNT] = {0};
  int cnt[SPEC_OP_COUNT] = {0};
  const int32_t sid = 0;
  int rc = SPEC_OK;
  for (int it = 0; it < iters && rc == SPEC_OK; ++it) {
    std::vector<hipEvent_t> ev;
    std::vector<int> ops;
    OpTimer tm{&ev, &ops};
    rc = upload_step(c, MODE_NO_COMMIT, 1, S, spans + (size_t)it * S, &sid);
    if (rc == SPEC_OK) rc = enqueue_forward(c, 1, S, &tm);
    if (rc == SPEC_OK) {
      hipError_t e = hipStreamSynchronize(c->st);
      for (size_t i = 0; e == hipSuccess && i + 1 < ev.size(); ++i) {
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, ev[i], ev[i + 1]);
        if (e == hipSuccess && ops[i] >= 0) {
          tot[ops[i]] += ms;
          if (it == 0) cnt[ops[i]]++;
        }
      }
      if (e != hipSuccess) rc = set_err(c, SPEC_EHIP, std::string("profiling: ") + hipGetErrorString(e));
    }
    for (auto e : ev) (void)hipEventDestroy(e);
  }
  trim_blocks(c, 0, c->len[0]);
  c->last_rows = S;
  if (rc != SPEC_OK) return rc;
  for (int op = 0; op < SPEC_OP_COUNT; ++op) {
    launches_out[op] = cnt[op];
    us_out[op] = cnt[op] ? (float)(tot[op] * 1000.0 / ((double)cnt[op] * iters)) : 0.0f;
  }
  return SPEC_OK;
}

int spec_time_op(spec_ctx* c, int op, int S, int reps, float* us_out) {
  if (!c || !us_out || reps <= 0) return c ? set_err(c, SPEC_EINVAL, "bad timing arguments") : SPEC_EINVAL;
  if ((op & 0xFF) < 0 || (op & 0xFF) >= SPEC_OP_COUNT) return set_err(c, SPEC_EINVAL, "unknown op class");
  if (S < 1 || S > SPEC_MAX_SPAN || S > c->lo.max_rows) return set_err(c, SPEC_EINVAL, "S must be in [1, 16]");
  STEP(check_ready(c));
  if (!c->live[0]) return set_err(c, SPEC_ESTATE, "timing before prefill");
  if (c->len[0] + S > c->lo.max_ctx) return set_err(c, SPEC_ECAPACITY, "cache length + span exceeds max_ctx");
  bool dirty = false;
  STEP(ensure_blocks(c, 0, c->len[0] + S, &dirty));
  if (dirty) STEP(upload_bt_row(c, 0));
  std::vector<int32_t> span((size_t)S, 0);
  const int32_t sid = 0;
  STEP(upload_step(c, MODE_NO_COMMIT, 1, S, span.data(), &sid));
  const bool per_layer = !(op == SPEC_OP_EMBED || op == SPEC_OP_LM);
  const int per_rep = per_layer ? c->lo.L : 1;
  // the embedding (which also resolves the rows' positions for the QKV
  // epilogue), one untimed pass, then the timed passes back to back
  if (op != SPEC_OP_EMBED) STEP(launch_op(c, SPEC_OP_EMBED, 0, 1, S));
  for (int l = 0; l < per_rep; ++l) STEP(launch_op(c, op, l, 1, S));
  hipEvent_t e0, e1;
  HIPCHK(c, hipEventCreate(&e0));
  HIPCHK(c, hipEventCreate(&e1));
  int rc = SPEC_OK;
  hipError_t e = hipEventRecord(e0, c->st);
  for (int r = 0; r < reps && rc == SPEC_OK && e == hipSuccess; ++r)
    for (int l = 0; l < per_rep && rc == SPEC_OK; ++l) rc = launch_op(c, op, l, 1, S);
  if (rc == SPEC_OK && e == hipSuccess) e = hipEventRecord(e1, c->st);
  if (rc == SPEC_OK && e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (rc == SPEC_OK && e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  trim_blocks(c, 0, c->len[0]);
  if (rc != SPEC_OK) return rc;
  if (e != hipSuccess) return set_err(c, SPEC_EHIP, std::string("timing: ") + hipGetErrorString(e));
  *us_out = ms * 1000.0f / (float)(reps * per_rep);
  return SPEC_OK;
}

int spec_measure_read_bw(const void* buf, size_t bytes, uint32_t* sink, int reps, void* hip_stream,
                         double* gbps_out) {
  if (!buf || !sink || !gbps_out || reps < 1 || bytes < (1u << 20) || bytes % 16 || !hip_stream)
    return SPEC_EINVAL;
  hipStream_t st = (hipStream_t)hip_stream;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus < 1)
    return SPEC_EHIP;
  const int grid = cus * 8;
  if (launch_stream_read(buf, bytes, sink, grid, st) != hipSuccess) return SPEC_EHIP;  // warm
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return SPEC_EHIP;
  }
  hipError_t e = hipEventRecord(e0, st);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch_stream_read(buf, bytes, sink, grid, st);
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess || ms <= 0.0f) return SPEC_EHIP;
  *gbps_out = (double)bytes * reps / (ms * 1e-3) / 1e9;
  return SPEC_OK;
}

int spec_measure_read_chain(const void* buf, size_t region_bytes, int n_regions, int grid, uint32_t* sink,
                            void* hip_stream, double* us_out) {
  if (!buf || !sink || !us_out || !hip_stream || region_bytes < 16 || region_bytes % 16 || n_regions < 1 ||
      grid < 1 || grid > 65535 || ((uintptr_t)buf & 15))
    return SPEC_EINVAL;
  hipStream_t st = (hipStream_t)hip_stream;
  const char* base = (const char*)buf;
  if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) return SPEC_EHIP;
  hipError_t e = hipSuccess;
  for (int r = 0; r < n_regions && e == hipSuccess; ++r)
    e = launch_stream_read(base + (size_t)r * region_bytes, region_bytes, sink, grid, st);
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(st, &g);
  if (e != hipSuccess || ec != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    return SPEC_EHIP;
  }
  hipGraphExec_t ge = nullptr;
  e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return SPEC_EHIP;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    (void)hipGraphExecDestroy(ge);
    return SPEC_EHIP;
  }
  e = hipGraphLaunch(ge, st);  // warm
  if (e == hipSuccess) e = hipEventRecord(e0, st);
  if (e == hipSuccess) e = hipGraphLaunch(ge, st);
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipGraphExecDestroy(ge);
  if (e != hipSuccess || ms <= 0.0f) return SPEC_EHIP;
  *us_out = (double)ms * 1000.0 / n_regions;
  return SPEC_OK;
}

int spec_op_bytes(const spec_model_desc* d, int op, int S, int ctx_len, double* bytes_out) {
  if (!d || !bytes_out || S < 1 || ctx_len < 0) return SPEC_EINVAL;
  const double H = d->hidden, hd = d->head_dim, DQ = (double)d->n_q_heads * hd, DK = (double)d->n_kv_heads * hd;
  const double F = d->ffn, V = d->vocab;
  // weight bytes per element: bf16 2; int4 0.5 plus one bf16 scale per 128
  const double wb = d->weight_format == SPEC_WFMT_INT4G128 ? 0.5 + 2.0 / 128.0 : 2.0;
  switch (op) {
    case SPEC_OP_EMBED: *bytes_out = S * H * 2.0; break;
    case SPEC_OP_QKV: *bytes_out = (DQ + 2 * DK) * H * wb + S * DK * 2 * 2.0; break;
    case SPEC_OP_ATTN: *bytes_out = (double)(ctx_len + S) * DK * 2 * 2.0; break;
    case SPEC_OP_O: *bytes_out = H * DQ * wb; break;
    case SPEC_OP_GATEUP: *bytes_out = 2 * F * H * wb; break;
    case SPEC_OP_DOWN: *bytes_out = H * F * wb; break;
    case SPEC_OP_LM: *bytes_out = V * H * wb; break;
    default: return SPEC_EINVAL;
  }
  return SPEC_OK;
}

// ------------------------------------------------------------ generation

}  // extern "C"

struct spec_gen {
  spec_ctx* c;
  spec_gen_params gp;
  int capacity, kcap, k;
  spec_ngram* ng;
  spec_governor* gov;  // governed loops only
  std::vector<int32_t> out;
  ~spec_gen() {
    spec_ngram_destroy(ng);
    spec_governor_destroy(gov);
  }
};

extern "C" {

int spec_gen_begin(spec_ctx* c, const int32_t* prompt, int n_prompt, int capacity, const spec_gen_params* gp,
                   spec_gen** res) {
  if (!c) return SPEC_EINVAL;
  if (!prompt || n_prompt <= 0 || capacity <= 0 || !gp || !res)
    return set_err(c, SPEC_EINVAL, "bad generation arguments");
  if (gp->spec && gp->draft_source != SPEC_DRAFT_NGRAM && !gp->ref_stream)
    return set_err(c, SPEC_EINVAL, "draft source needs ref_stream");
  spec_gen* g = new (std::nothrow) spec_gen;
  if (!g) return set_err(c, SPEC_ECAPACITY, "out of host memory");
  g->c = c;
  g->gp = *gp;
  g->capacity = capacity;
  g->kcap = std::max(1, std::min(gp->fixed_k > 0 ? gp->fixed_k : gp->k_cap, SPEC_MAX_SPAN - 1));
  g->k = gp->fixed_k > 0 ? std::min(gp->fixed_k, SPEC_MAX_SPAN - 1) : 1;
  g->ng = nullptr;
  g->gov = nullptr;
  int rc = SPEC_OK;
  if (gp->spec && gp->draft_source == SPEC_DRAFT_NGRAM)
    rc = spec_ngram_create(gp->n_min, gp->n_max, n_prompt + capacity + 1, &g->ng);
  if (rc == SPEC_OK && gp->spec && gp->governed) rc = spec_governor_create(nullptr, &g->gov);
  int32_t g0 = 0;
  if (rc == SPEC_OK) rc = spec_prefill(c, prompt, n_prompt, &g0);
  if (rc == SPEC_OK && g->ng) rc = spec_ngram_append(g->ng, prompt, n_prompt);
  if (rc == SPEC_OK && g->ng) rc = spec_ngram_append(g->ng, &g0, 1);
  if (rc != SPEC_OK) {
    delete g;
    return rc;
  }
  g->out.reserve((size_t)capacity);
  g->out.push_back(g0);
  *res = g;
  return SPEC_OK;
}

int spec_gen_step(spec_gen* g, int rounds, spec_gen_stats* gs) {
  using clk = std::chrono::steady_clock;
  if (!g || !gs || rounds < 0) return SPEC_EINVAL;
  spec_ctx* c = g->c;
  const spec_gen_params& gp = g->gp;
  int32_t span[SPEC_MAX_SPAN], am[SPEC_MAX_SPAN];
  const auto t0 = clk::now();
  double in_verify = 0.0;
  int done = 0;
  while (done < rounds && (int)g->out.size() < g->capacity) {
    const auto tr = clk::now();
    const int n = (int)g->out.size();
    int kd = 0;
    // a governed loop drafts only when its governor says so
    const bool draft = gp.spec && (!g->gov || spec_governor_should_draft(g->gov) == 1);
    if (draft) {
      const int want = std::max(0, std::min(g->k, g->capacity - n - 1));
      if (gp.draft_source == SPEC_DRAFT_NGRAM) {
        kd = spec_ngram_propose(g->ng, want, span + 1);
        if (kd < 0) return set_err(c, kd, "n-gram propose");
      } else {
        kd = want;
        for (int i = 0; i < kd; ++i) {
          const int32_t t = gp.ref_stream[n + i];
          span[1 + i] = gp.draft_source == SPEC_DRAFT_WRONG ? (t + 1) % c->lo.V : t;
        }
      }
    }
    span[0] = g->out.back();
    int32_t m = 0;
    const int p = c->len[0];
    const auto tv = clk::now();
    STEP(spec_verify(c, span, kd, am, &m));
    in_verify += std::chrono::duration<double>(clk::now() - tv).count();
    gs->forwards++;
    gs->drafted += kd;
    gs->accepted += m;
    gs->accept_hist[m]++;
    gs->forwards_by_span[kd + 1]++;
    int commit = m + 1;
    if (commit > g->capacity - n) {  // not expected: drafts never pass the budget
      commit = g->capacity - n;
      STEP(spec_rewind(c, p + commit));
    }
    for (int i = 0; i < commit; ++i) g->out.push_back(am[i]);
    if (g->ng) STEP(spec_ngram_append(g->ng, am, commit));
    if (draft && gp.fixed_k <= 0) g->k = spec_adapt_k(g->k, kd, m, g->kcap);
    if (g->gov) {
      if (!draft) gs->plain_steps++;
      const double sec = std::chrono::duration<double>(clk::now() - tr).count();
      STEP(spec_governor_record(g->gov, draft ? 1 : 0, commit, m, sec));
    }
    ++done;
  }
  const double dt = std::chrono::duration<double>(clk::now() - t0).count();
  gs->decode_s += dt;
  gs->host_s += dt - in_verify;
  return done;
}

int spec_gen_tokens(spec_gen* g, int32_t* out, int cap) {
  if (!g || (cap > 0 && !out) || cap < 0) return SPEC_EINVAL;
  const int n = std::min(cap, (int)g->out.size());
  if (n > 0) memcpy(out, g->out.data(), sizeof(int32_t) * (size_t)n);
  return (int)g->out.size();
}

int spec_gen_governor_stats(spec_gen* g, spec_governor_stats* out) {
  if (!g || !out || !g->gov) return SPEC_EINVAL;
  return spec_governor_get_stats(g->gov, out);
}

int spec_gen_end(spec_gen* g) {
  delete g;
  return SPEC_OK;
}

int spec_generate(spec_ctx* c, const int32_t* prompt, int n_prompt, int n_tokens, const spec_gen_params* gp,
                  int32_t* out, spec_gen_stats* gs) {
  using clk = std::chrono::steady_clock;
  if (!c) return SPEC_EINVAL;
  if (!out || !gs) return set_err(c, SPEC_EINVAL, "bad generation arguments");
  memset(gs, 0, sizeof(*gs));
  const auto t0 = clk::now();
  spec_gen* g = nullptr;
  STEP(spec_gen_begin(c, prompt, n_prompt, n_tokens, gp, &g));
  gs->prefill_s = std::chrono::duration<double>(clk::now() - t0).count();
  const int rc = spec_gen_step(g, n_tokens, gs);
  if (rc >= 0) spec_gen_tokens(g, out, n_tokens);
  spec_gen_end(g);
  return rc < 0 ? rc : SPEC_OK;
}

}  // extern "C"
