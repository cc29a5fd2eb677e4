// internal.h -- kernel parameter blocks shared by the libspecv runtime and its
// gfx950 kernels.  Not part of the public ABI (include/specv.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

constexpr int kMaxRows = 128;  // rows per forward (the library-wide limit of the C ABI)

// Step modes, read by the accept stage from device memory so one captured
// graph per shape serves all three.
enum StepMode { MODE_VERIFY = 0, MODE_COMMIT_ALL = 1, MODE_NO_COMMIT = 2 };

// GEMM epilogues.
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LM = 3 };

// Device step block: written by one host-to-device copy before each forward.
struct StepDev {
  int32_t mode;
  int32_t n_seq;
  int32_t span;      // rows per sequence (S)
  int32_t pad;
  float temp;        // 0: greedy (argmax rows); > 0: every row draws its token at this temperature
  uint32_t seed_lo, seed_hi;  // the draws' seed (Philox key)
  int32_t pad2;
  // followed by tokens[max_rows], seq_ids[max_rows] and kd[max_rows] (the
  // drafts each sequence really proposed; its span rows past 1 + kd are padding)
};

// Packed bf16 weights: fragments of 16 output rows x 32 inputs, 1 KiB each,
// stored lane-major in the order the MFMA B operand is read:
//   frag(t, s)[lane] = W[16t + lane%16][32s + 8*(lane/16) .. +8]
// at ((t * (K/32) + s) * 64 + lane) * 16 bytes.
inline size_t packed_bf16_bytes(int N, int K) { return (size_t)N * K * 2; }

// Weight formats of the GEMMs (the embedding is always bf16).
enum WFmt { FMT_BF16 = 0, FMT_INT4 = 1 };

// Packed int4 group-128 weights: per 16-row tile t and 128-input group g one
// 1 KiB fragment, lane-major in the order the MFMA B operand is read:
//   frag(t, g)[lane] dword d (d = 0..3, the four 32-input steps of the group)
//   holds W[16t + lane%16][128g + 32d + 8*(lane/16) + e], e = 0..7, as offset
//   nibbles u = q + 8 at bit 4*(e/2) + 16*(e%2),
// so ((dword >> 4j) & 0x000F000F) holds the pair (e = 2j, 2j+1) in the two
// halves of a packed fp16 pair.  Fragments at ((t * (K/128) + g) * 64 + lane)
// * 16 bytes; then the scales, bf16 [N/16][16][K/128] (tile, row, group).
inline size_t packed_int4_frag_bytes(int N, int K) { return (size_t)N * K / 2; }
inline size_t packed_int4_bytes(int N, int K) {
  return packed_int4_frag_bytes(N, K) + (size_t)N * (K / 128) * 2;
}

struct GemmParams {
  const void* W;         // packed fragments (bf16: [N/16][K/32][64] x 16 B; int4: [N/16][K/128][64] x 16 B)
  const uint16_t* scales;// int4 only: bf16 group scales [N/16][16][K/128]
  int N, K, R;           // outputs, inputs, rows
  int nslices;           // K split into nslices slices of NK*32 inputs
  const float* A;        // activation rows [R][lda] (fp32)
  const _Float16* A16;   // or, for the LDS-staged and phased one-pass residual GEMMs, the same rows
                         // already rounded to fp16 ([R][lda]), else null
  int lda;
  const void* Af;        // or, bf16 only: A prepared by k_prep (fp16 fragments), else null
  const float* ss;       // RMSNorm: per-row partial sums of squares [R][ss_n], or null
  int ss_n;
  const float* gain;     // RMSNorm gain [K]
  float eps, inv_dim;
  float* part;           // split partial sums [nslices][R][N]
  unsigned* cnt;         // arrival counter per 64-column block
  // EPI_QKV
  float* q;              // [R][n_q*hd] rotated queries (recurrent layers: unrotated), or
  _Float16* q16;         // an attention layer's rotated queries rounded to fp16 (what attention reads)
  _Float16* kpool;       // this layer's K blocks [n_blocks][n_kv][16][hd]
  _Float16* vpool;       // this layer's V blocks [n_blocks][n_kv][hd][16]
  const int32_t* bt;     // block tables [max_seqs][bt_stride]
  int bt_stride;
  const int32_t* kv_len; // cache length per sequence (read-only here)
  const int32_t* seq_ids;// [n_seq]
  int S, n_q, n_kv, hd;
  const float* rope;     // [max_ctx][hd/2][2] = cos, sin
  const int32_t* rowinfo;// [R][2]: each row's absolute position and its KV block (k_embed)
  int ring_nb, ring_w;   // sliding-window layer: the KV rows go to the sequence's ring of ring_w
                         // slots (ring_nb blocks): block seq * ring_nb + (pos % ring_w) / 16; else 0
  float* rec_kv;         // recurrent layer: unrotated keys and values [R][2][n_kv*hd] (queries
                         // unrotated into q), no cache rows; else null
  // EPI_RESID
  float* x;              // residual [R][N]
  float* ss_out;         // [R][N/64] partial sums of squares of the new residual
  // EPI_SWIGLU
  float* h;              // [R][N/2]
  _Float16* h16;         // or null: h also rounded to fp16 (the down projection's A16)
  void* af_out;          // or null: h also as the next GEMM's prepared A (k_prep's layout)
  // EPI_LM
  unsigned long long* argkey; // per-row packed (value, index) maxima, zero between forwards
  unsigned* lm_cnt;           // arrival counter over all column blocks
  int32_t* status;            // bit 0: NaN logit seen
  float* logits;              // [R][N] or null
  const int32_t* tokens;      // [R] span tokens
  const int32_t* kd;          // [n_seq] drafts per sequence (rows past 1 + kd[b] are padding)
  const int32_t* mode;        // StepDev::mode
  const StepDev* step;        // the step block: sampling temperature and seed
  int32_t* rec_slot;          // or null: per sequence, the recurrent state slot (set * 16 + row, -1 =
                              // zero) committed by the accept stage
  int32_t* result;            // [1 + n_seq*(S+1)]: status, then (m, a0..a(S-1)) per sequence
  int32_t* kv_len_w;          // cache lengths, advanced by the accept stage
  int n_seq;
};

struct AttnParams {
  const _Float16* q;     // [R][n_q*hd] rotated queries, fp16 (the QKV epilogue's rounding)
  const int32_t* rowinfo;// [R][2] (k_embed): row b*S's position is sequence b's cache length
  const int32_t* slotbt; // [n_seq][bt_stride] (k_embed): sequence b's block table row
  const _Float16* kpool; // [n_blocks][n_kv][16][hd]
  const _Float16* vpool; // [n_blocks][n_kv][hd][16]
  int bt_stride;
  int S, n_seq, n_q, n_kv;
  float scale;
  int max_splits;        // grid.x: 256-key splits of the longest context
  float* part;           // [n_kv][max_splits][R*G][2 + hd]: (max, sum, unnormalised o)
  unsigned* cnt;         // [n_seq][n_kv][tile groups] arrival counters of the fused merge, zero between launches
  float* out;            // [R][n_q*hd]
  _Float16* out16;       // or null: out also rounded to fp16 (the O projection's A16)
  void* af_out;          // or null: out also as the O GEMM's prepared A (k_prep's layout)
  int n_qt;              // query tiles per sequence: ceil(S * n_q / n_kv / 16)
  int tpw;               // query tiles per workgroup (1..n_qt), taken one after another
  int fuse;              // short contexts: the last split of a tile merges it in k_attn
  // sliding-window layer (win > 0): row at position t attends keys [t - win + 1, t],
  // read from the sequence's ring (block seq_ids[b] * ring_nb + (position / 16) % ring_nb);
  // grid.x covers grid_splits splits from the first one the window touches
  int win, ring_nb, ring_w, grid_splits;
  const int32_t* seq_ids;
};
// The attention merges its splits in the same kernel when every context of
// the step (cache + span) spans at most attn_fuse_splits(hd) splits of 256
// keys: the last split of each query tile to finish then merges the tile's
// columns itself, keeping the splits' (max, sum) in its LDS.
constexpr int attn_fuse_splits(int hd) { return hd >= 32 ? 64 : 32; }

// A recurrent (delta-rule) layer's step over the span rows of each sequence.
struct RecParams {
  const float* q;        // [R][n_q*hd] unrotated queries
  const float* kv;       // [R][2][n_kv*hd] unrotated keys, values
  float* snap;           // [max_seqs][2 sets][16 rows][n_kv][hd (v)][hd (k)]: the state after each row
  const int32_t* slot;   // [max_seqs]: the committed state (set * 16 + row), or -1 for the zero state
  const int32_t* seq_ids;
  float* out;            // [R][n_q*hd]
  void* af_out;          // or null: out also as the O GEMM's prepared A
  int S, n_seq, n_q, n_kv;
  float beta;
};

struct EmbedParams {
  const uint16_t* emb;   // [V][H] bf16
  const int32_t* tokens; // [R]
  float* x;              // [R][H]
  float* ss;             // [R][H/16]
  int H;
  // each row's position and KV block, for every layer's QKV epilogue:
  // rowinfo[2r] = kv_len[seq_ids[r/S]] + r%S, rowinfo[2r+1] = its block
  const int32_t* seq_ids;
  const int32_t* kv_len;
  const int32_t* bt;
  int bt_stride, S;
  int32_t* rowinfo;
  int32_t* slotbt;       // [n_seq][bt_stride]: the block table rows of the step's sequences, by slot
};

// Launchers (kernels.hip).  All return hipSuccess or the launch error.
hipError_t launch_gemm(const GemmParams& p, int nk, int epi, int fmt, hipStream_t st);
// Above 16 rows (bf16, prepared A in p.Af): the many-row GEMM over ns K
// slices (ns > 1: slice partials in p.part, summed by a gather kernel; the
// LM head needs ns = 1) with ct (1 or 2) 16-column tiles per wave.
hipError_t launch_gemm_big(const GemmParams& p, int ns, int ct, int epi, hipStream_t st);
#ifndef SPECV_BIG_PD1
#define SPECV_BIG_PD1 8  // steps in flight, one tile per wave
#endif
#ifndef SPECV_BIG_PD2
#define SPECV_BIG_PD2 4  // two tiles per wave
#endif
// Prepare A for the many-row GEMM (kernels.hip: k_prep): the RMSNorm (when
// p.ss is set) and the fp16 rounding of every row once, in the 16x16x32 MFMA
// A-operand order, into af: ceil(R/16) * 16 * K * 2 bytes.
hipError_t launch_prep_a(const GemmParams& p, void* af, hipStream_t st);
// One-pass GEMM for R <= 16 (kernels.hip: k_mm, k_mm1): nw waves split K
// into nw parts of spw 32-input steps, summed in groups of gp parts (gp = 1
// or nw: the plain part order); nbuf 1 or 2: blocks of ct 16-column tiles
// walked by at most max_grid workgroups with nbuf weight buffers; nbuf 0:
// one tile per workgroup in ct phases.  With gp = 1 or nw numerically
// identical to launch_gemm with nk = spw (nslices = nw).
bool mm_supported(int epi, int nw, int spw, int ct, int nbuf, int gp);
// The residual one-pass GEMM for at most rl rows with A staged in LDS
// (kernels.hip: k_mm1l); compiled for (nw, spw, rl) = (16, 19, 8) (down) and
// (8, 16, 4) (O); rows up to rl take the smallest staging that holds them.
hipError_t launch_mm1l(const GemmParams& p, int nw, int spw, int rl, hipStream_t st);
// The int4 one-pass GEMM for at most four rows (kernels.hip: k_mmq): waves
// own the K parts of the int4 split-K kernel with nk-step slices, so the two
// agree bit for bit; compiled for K / (32 nk) waves of nk / 4 groups in
// {10 x 4, 16 x 4, 1 x 1}.
bool mmq_supported(int K, int nk, int epi);
hipError_t launch_mmq(const GemmParams& p, int nk, int epi, int max_grid, hipStream_t st);
bool mmqr_plan(int K, int* nw, int* gpw, int* parts);
hipError_t launch_mmqr(const GemmParams& p, int epi, int max_grid, hipStream_t st);
hipError_t launch_mm(const GemmParams& p, int nw, int spw, int ct, int nbuf, int gp, int max_grid, int epi,
                     hipStream_t st);
hipError_t launch_attn(const AttnParams& p, int hd, hipStream_t st);
// One workgroup per (kv head, sequence); the rows of each span in order.
hipError_t launch_recur(const RecParams& p, int hd, hipStream_t st);
hipError_t launch_embed(const EmbedParams& p, int R, hipStream_t st);
// Repack canonical bf16 [rows][cols] as fp16 into fragments of a fused
// matrix whose row for source row s is map(s): kind 0 identity + row0, kind
// 1 RoPE pair interleave within heads of hd rows (+ row0), kind 2 row 2s +
// row0.  A value beyond the fp16 range sets *overflow (device word) to 1.
hipError_t launch_pack_bf16(const uint16_t* src, int rows, int cols, void* dst, int kind, int row0,
                            int hd, uint32_t* overflow, hipStream_t st);
// The same for canonical int4 group-128 (q4 bytes [rows][cols/2], low nibble
// = even column; bf16 scales [rows][cols/128]) into int4 fragments and the
// matrix's scale block.
hipError_t launch_pack_int4(const uint8_t* q4, const uint16_t* scales, int rows, int cols, void* dst_frag,
                            uint16_t* dst_scales, int kind, int row0, int hd, hipStream_t st);
hipError_t launch_fill_u32(void* dst, uint32_t value, size_t count, hipStream_t st);
// Stream `bytes` (a multiple of 16) from src with non-temporal 16-byte loads
// over `grid` workgroups; sink: 256 words of device scratch.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t st);

// Row of the fused QKV matrix holding source row s of a Q or K projection:
// the pair (d, d + hd/2) of a head lands on adjacent rows (2d, 2d+1).
__host__ __device__ inline int rope_pair_row(int s, int hd) {  // source row -> interleaved row
  const int h = s / hd, d = s % hd, half = hd / 2;
  return h * hd + (d < half ? 2 * d : 2 * (d - half) + 1);
}

}  // namespace specv
