// Internal declarations shared by the C-ABI layer (abi.cpp) and the HIP
// kernels (kernels.hip).  Not part of the public interface.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace atd {

constexpr int kMaxTables = 16;
constexpr int kMaxLayers = 64;
constexpr int kGemvMaxRows = 2;      // rows a GEMV launch handles at once
constexpr int kArgmaxChunk = 4096;   // logits per argmax block
constexpr int kAttnWavesMax = 8192;   // largest split-count target of a launch
constexpr int kAttnWavesFew = 1024;   // split-count target of a launch of at most 4 rows
// In a launch of at most 4 rows, a row of at most this many keys takes one
// block of four splits (no merge across blocks; measured: ASR shape +0.9%,
// 0.6B frame loop +1.2%, 1.7B Talker + Code Predictor frames +0.9%)
constexpr int kAttnOneBlockKeys = 256;
constexpr int kAttnSplitsMax = 256;   // most splits of one (row, KV head)
constexpr int kAttnMinChunk = 16;     // fewest keys per split

#if defined(__HIP__)
#define ATD_HD __host__ __device__
#else
#define ATD_HD
#endif

// Keys per attention split for a row whose valid length is len, in a launch
// of M rows over Hkv KV heads aiming at `waves` splits in total: every row
// gets the same number of splits (all waves busy), each at least
// kAttnMinChunk keys, a multiple of 16; in a launch of at most 4 rows a row
// of at most kAttnOneBlockKeys keys gets four (one block).  Depends on (len,
// M, Hkv, waves)
// only, never on the cache capacity (results do not change when a bucket
// grows).
inline ATD_HD int attn_splits_per_head(int M, int Hkv, int waves) {
  const int per = waves / (M * Hkv);
  return per < 1 ? 1 : (per > kAttnSplitsMax ? kAttnSplitsMax : per);
}
inline ATD_HD int attn_chunk(int len, int M, int Hkv, int waves) {
  if (waves <= kAttnWavesFew && len <= kAttnOneBlockKeys) {
    const int c = (((len + 3) / 4) + 15) & ~15;
    return c < kAttnMinChunk ? kAttnMinChunk : c;
  }
  const int per = attn_splits_per_head(M, Hkv, waves);
  int c = (len + per - 1) / per;
  c = (c + 15) & ~15;
  return c < kAttnMinChunk ? kAttnMinChunk : c;
}

// Upper bound of the split count of any row of length <= max_len.
inline int attn_max_splits(int max_len, int M, int Hkv, int waves) {
  const int a = (max_len + kAttnMinChunk - 1) / kAttnMinChunk;
  const int b = attn_splits_per_head(M, Hkv, waves);
  return a < b ? a : b;
}

// How the rows of a launch map to (slot, position):
//  kRowsStep:    row m -> slot slot_list[row0 + m] (or slot0 + row0 + m when
//                there is no list) at that slot's current position
//  kRowsPrefill: row m -> slot slot0 at position row0 + m
enum RowMode { kRowsStep = 0, kRowsPrefill = 1 };

struct RowMap {
  int mode;
  int slot0;
  int row0;       // rows of this launch are rows row0 .. of the call
  int rope_rows;  // 1: the RoPE tables hold one row per call row (row0 + m),
                  // built from rotary positions; 0: indexed by position
  const int32_t* slot_list = nullptr;  // device [rows of the call]: slot of each
                                       // step row, or null (contiguous slots)
};

// Slot of step row r (a row of the whole call).
inline ATD_HD int step_slot(const RowMap& rm, int r) {
  return rm.slot_list ? rm.slot_list[r] : rm.slot0 + r;
}

// Host slot list -> device (up to kSlotListChunk entries per launch, passed by
// value, so the copy needs no staging buffer and can be captured in a graph).
constexpr int kSlotListChunk = 256;
struct SlotListArgs {
  int32_t v[kSlotListChunk];
  int n, off;
};

// ---------------------------------------------------------------- rows/KV
struct SlotTables {
  void** kv;        // device [max_slots][L][2] cache pointers (K, V)
  int* pos;         // device [max_slots] next write position
  int* cap;         // device [max_slots] capacity (rows)
  int L;
};

struct RopeArgs {
  const float* qkv;   // [M, (Hq + 2 Hkv) D]
  float* q_out;       // [M, Hq, D]
  const float* q_norm;
  const float* k_norm;
  float eps;
  const float* cos_t; // [max_ctx, D/2]
  const float* sin_t;
  SlotTables st;
  RowMap rows;
  int layer, M, Hq, Hkv, D, qk_norm;
};

// ---------------------------------------------------------------- GEMV
enum GemvEpilogue { kEpiStore = 0, kEpiResidual = 1, kEpiSwiglu = 2 };

// Weight storage of a GEMV: dense float32 / bf16, or block-quantized codes
// (int8, or 4-bit pairs) with one fp16 scale per kQBlock weights of a row.
// kWBF16NT: bf16 weights streamed with the nontemporal cache policy (for
// decoders whose weights exceed the memory-side cache, kMallBytes)
enum WeightType { kWF32 = 0, kWBF16 = 1, kWQ8 = 2, kWQ4 = 3, kWBF16NT = 4 };
constexpr size_t kMallBytes = (size_t)256 << 20;
constexpr int kQBlock = 32;

struct GemvArgs {
  const void* W[3];       // row segments [rows_s, K]; segment s ends at seg_end[s]
  const uint16_t* S[3];   // fp16 block scales [rows_s, K / kQBlock] (quantized types)
  const uint16_t* S2;     // scales of W2
  const float* bias[3];   // per-segment bias or null (kEpiStore only)
  int seg_end[3];
  const void* W2;         // up-projection [N, K] (kEpiSwiglu)
  const float* x;         // input rows [M, ldx]
  int ldx;
  const float* gain;      // RMSNorm gain [K] when the input is normalised
  float eps;
  float* out;             // output rows [M, ldo]
  int ldo;
  float* y_out;           // normalised input rows [M, K] (block 0 writes), or null
  int K, N, M;
};





// Weights that later launches read, pulled into the L2 of the XCD whose
// compute units will read them.  The L2 of each XCD keeps its lines across
// kernel boundaries, and workgroup w of every launch runs on XCD w % 8
// (measured), so block b of a later 1-D launch finds on its own XCD whatever
// a workgroup on XCD b % 8 loaded.  Region r describes such a launch: its
// block b reads bytes [b * bb, (b + 1) * bb) of base[r] (bb a multiple of
// 16), and the first nblk[r] blocks are covered.  The loads only warm the
// cache: nothing is computed from them.
constexpr int kPfRegions = 4;
struct L2Prefetch {
  const char* base[kPfRegions];
  size_t bb[kPfRegions];
  int nblk[kPfRegions];
  int nreg;     // regions in use, 0 = no prefetch
};
// Bytes a step attention launch prefetches: 3 of the 4 MiB of each XCD's L2
// (measured on the 1.7B step, O projection + gate/up prefix: 16 MiB 952,
// 24 MiB 959, 28 MiB 939, 32 MiB 940 tokens/s against 926 without).
constexpr size_t kL2PrefetchBytes = (size_t)24 << 20;
// Prefetch workgroups for the whole budget: a launch whose slice has fewer
// (gx * Hkv of them) prefetches proportionally less, so that each
// workgroup's share, and the time it takes, stay the same.
constexpr int kPfWorkgroups = 256;

struct AttnArgs {
  // fused (decode steps): q and the new k/v row come raw from qkv and get the
  // QK norm + RoPE here; the last split's wave appends the new row to the
  // cache.  Otherwise (prefill) q is the rotated q_out and every row is
  // already in the cache.
  int fused;
  const float* qkv;   // [M, (Hq + 2 Hkv) D] raw projections (fused)
  const float* q_norm;
  const float* k_norm;
  int qk_norm;
  float eps;
  const float* cos_t; // [max_ctx, D/2]
  const float* sin_t;
  const float* q;     // [M, Hq, D] rotated queries (not fused)
  SlotTables st;
  RowMap rows;
  int layer, M, Hq, Hkv, nsplit_max;   // nsplit_max: split stride of the partials
  int waves;                           // split-count target of the launch (attn_chunk)
  // single-slot launches: the slot's cache rows of this layer and capacity,
  // passed directly so no pointer table is read (null: use st)
  void* k_direct;
  void* v_direct;
  int cap_direct;
  float scale;
  float* pml;         // [M, Hq, nsplit_max, 2] running max and sum of each block
  float* pacc;        // [M, Hq, nsplit_max, D] (block b of a row at index b)
  int* ticket;        // [M, Hkv] arrivals of a row's blocks (zero between launches)
  float* o;           // [M, Hq * D] attention output
  uint16_t* o_hi;     // or, when set, bf16 hi/lo parts of o: [M, Hq * D]
  uint16_t* o_lo;
  int o_frag;         // o_hi / o_lo in MFMA-fragment order (frag_off; M <= 64)
  // deferred merge: the blocks of a (row, KV head) write their partial states
  // and a second launch (k_attn_merge) merges them, in place of the
  // last-arriving block (no prefetch slice with it)
  int defer;
  // with pf.nreg > 0 the launch has one more z slice (z = M) whose
  // workgroups only run the prefetch
  L2Prefetch pf;
};

struct EmbedArgs {
  const void* tab[kMaxTables];
  int vocab[kMaxTables];
  int G;
  const int32_t* tok;   // [M, G]
  const float* extra;   // [M, h] or null
  const int32_t* extra_row;  // device row index: extra starts (*extra_row) rows further, or null
  float* out;           // [M, h]
  int h, M;
};

// Generation controls of a token choice: suppressed tokens, and eos while the
// choice index is below min_new, read as -inf; a stopped row (eos_step >= 0)
// returns eos.  The choice index is step0 + *step_base + *step_ctr (either
// pointer may be null).
struct ChoiceCtl {
  const uint32_t* suppress = nullptr;   // [B, nwords] or null
  int eos = -1;
  int min_new = 0;
  int step0 = 0;
  const int32_t* step_base = nullptr;   // device value added to step0, or null
  const int32_t* step_ctr = nullptr;    // device counter added too, or null
  int32_t* eos_step = nullptr;          // [B] or null (no stop)
};

struct ArgmaxArgs {
  const float* z;      // [B, V]
  int B, V;
  uint32_t* seen;      // [B, nwords] or null
  int nwords;
  float penalty;
  int32_t* tok;
  float* margin;
  float* part;         // [B, nblk, 3]
  int nblk;
  ChoiceCtl ctl;
};

// top-k sampling: one 1024-thread workgroup selects from up to kSampleChunk
// values (8 per thread); longer rows are cut into chunks whose top-k
// candidates a second workgroup selects from
constexpr int kTopKMax = 256;
constexpr int kSampleThreads = 1024;
constexpr int kSamplePerThread = 8;
constexpr int kSampleChunk = kSampleThreads * kSamplePerThread;

inline int sample_blocks(int V) { return (V + kSampleChunk - 1) / kSampleChunk; }

struct SampleArgs {
  const float* z;        // [B, V]
  int B, V;
  uint32_t* seen;        // [B, nwords] or null
  int nwords;
  float penalty;
  int k;                 // 1..kTopKMax, <= V
  float temperature;     // > 0
  float top_p;           // (0, 1]
  const float* u;        // row b draws u[(u_row ? *u_row : 0) * u_stride + b]
  const int32_t* u_row;  // device index or null
  int u_stride;
  int32_t* tok;          // [B]
  uint2* part;           // [B, nblk, k] candidates (order key, index) when nblk > 1
  int nblk;              // sample_blocks(V)
  ChoiceCtl ctl;
};

struct KvCopyArgs {
  const void* src[2 * kMaxLayers];
  void* dst[2 * kMaxLayers];
  int n;               // number of buffers (2 L)
  int Hkv, D, rows, s_old, s_new, elem_bytes;
};

// ---------------------------------------------------------------- MFMA path (M >= kMmaMinRows)
// Fewest rows a call takes the matrix-core path with.  Measured on the 1.7B
// shape (bf16 cache, context 1000), ms per step of M streams, matrix-core /
// vector path: 3 rows 1.98 / 1.89, 4 rows 1.95 / 1.93, 6 rows 2.30 / 2.94,
// 8 rows 2.37 / 3.71 (the vector path streams the weights once per 2 rows).
constexpr int kMmaMinRows = 5;
// Activations enter a GEMM as a bf16 pair hi + lo (hi = bf16(v), lo =
// bf16(v - hi)), so the products keep ~16 bits of the float32 input while the
// bf16 weights are used exactly; each float32 activation is split into bf16
// hi + lo parts as it is staged, so the products carry ~16 mantissa bits.
constexpr int kMmaRows = 64;     // rows per GEMM row tile (and per decode-step chunk)
constexpr int kMmaPrefillRows = 512;   // most rows of one layer-major prefill chunk
constexpr int kMmaBlockN = 64;   // weight rows per workgroup (16 per wave)
constexpr int kMmaCh = 64;       // K per pipeline stage
constexpr int kMmaCUs = 256;     // compute units of the part
constexpr int kSsCols = 16;      // columns per partial sum of squares (one MFMA column block)

// K per split of the GEMM of an [N, K] weight over `tiles` row tiles (a
// multiple of kMmaCh): the fewest splits that give every compute unit a
// workgroup and keep a split within 16 stages, raised (up to 4x) to a whole
// number of workgroups per unit when one exists, so that no partial round of
// workgroups trails the rest (measured on the 1.7B shapes)
inline int mma_kc(int N, int K, int tiles = 1) {
  const int nb = (N + kMmaBlockN - 1) / kMmaBlockN * tiles;
  // at most 16 stages per split: the stage counts the GEMM kernel has fully
  // unrolled forms for
  const int kmin = (K + 16 * kMmaCh - 1) / (16 * kMmaCh);
  const int kfill = (kMmaCUs + nb - 1) / nb;
  const int k0 = kfill > kmin ? kfill : kmin;
  int ks = k0;
  for (int k = k0; k <= 4 * k0; ++k)
    if ((nb * k) % kMmaCUs == 0) {
      ks = k;
      break;
    }
  long kc = (K + ks - 1) / ks;
  kc = (kc + kMmaCh - 1) / kMmaCh * kMmaCh;
  return (int)(kc < K ? kc : (K + kMmaCh - 1) / kMmaCh * kMmaCh);
}
inline int mma_ks(int N, int K, int tiles = 1) {
  const int kc = mma_kc(N, K, tiles);
  return (K + kc - 1) / kc;
}

struct GemmArgs {
  const uint16_t* hi;  // activations as bf16 hi + lo parts [mrows, K]; rows >= M may
  const uint16_t* lo;  // hold anything (each output row depends on its own row only)
  const void* W[3];    // bf16 row segments [rows_s, K]
  int seg_end[3];
  int K, N;            // K multiple of 32
  int kc, ks;          // K per split (multiple of kMmaCh) and number of splits
  int mrows;           // rows of the call, rounded up to row tiles of kMmaRows
  float* part;         // [ks, mrows, N]
};

enum ReduceEpilogue { kRedStore = 0, kRedResidual = 1, kRedSwiglu = 2 };

// GEMM of one 64-row tile of decode rows with the split-K reduction and the
// epilogue in the same launch (k_gemm_dec).  Epilogues: kDecParts leaves the
// split sums in part [ks, kMmaRows, N] for a later reduction; kDecStore writes
// out = inv_m * sum + bias; kDecResidual adds the sum into x (out) and leaves
// x * gain as the next GEMM's hi / lo input and kSsCols-column sums of squares
// of x; kDecSwiglu (N = 2 F: W[0] gate rows, W[1] up rows) leaves
// silu(inv_m g) * inv_m u as hi / lo.
enum DecEpilogue { kDecParts = 0, kDecStore = 1, kDecResidual = 2, kDecSwiglu = 3 };

// Offset of element (row r, column k) of a 64-row activation tile held in
// MFMA-fragment order: [k / 32][r / 16][(k % 32) / 8][r % 16][k % 8], so that
// the A-operand fragment of a 16x16x32 MFMA (lane 16 g + i: row i, columns
// 8 g .. 8 g + 7 of a 32-wide step) is one contiguous 1 KB run.  A wave reads
// such runs from L2 at about three times the rate of the same fragments out
// of row-major rows (16 rows x 64 bytes per load).
inline ATD_HD size_t frag_off(int r, int k) {
  return ((size_t)((k >> 5) * 4 + (r >> 4)) * 64 + ((k >> 3) & 3) * 16 + (r & 15)) * 8 + (k & 7);
}
constexpr int kDecKStep = 32;         // K per MFMA step
constexpr int kDecWaves = 8;          // waves per workgroup
constexpr int kDecMaxSteps = 16;      // most K steps per wave (kc <= 16 * 8 * 32)

// Weights of the decode GEMMs in MFMA B-operand order: 16-row blocks, each
// [K / 32][512] bf16 with the fragment of K step s at s * 512 (lane 16 g + i:
// row i, columns 32 s + 8 g .. + 7), so that a wave reads a fragment as one
// contiguous 1 KB run (the same fragment out of row-major rows is 16 runs of
// 64 bytes, 4 KB apart at K = 2048, measured at ~3.3 against ~4.3 TB/s).
// Block b holds rows 16 b .. 16 b + 15 of the matrix (rows past N zero); in
// SwiGLU order block 4 t + j holds gate rows 32 t + 16 j .. (j < 2) or up
// rows 32 t + 16 (j - 2) .. (j >= 2).
inline ATD_HD size_t bfrag_blocks(int N, bool swiglu) {
  return swiglu ? (size_t)(N / 2 + 31) / 32 * 4 : (size_t)(N + 15) / 16;
}
struct SwizzleArgs {
  const uint16_t* src[3];   // row segments (SwiGLU: gate [F, K], up [F, K])
  int seg_end[3];
  int N, K;                 // N rows (SwiGLU: 2 F); K a multiple of 32
  int swiglu;
  uint16_t* dst;            // bfrag_blocks(N, swiglu) * K * 16 elements
};

struct DecGemmArgs {
  const uint16_t* hi;   // activations as bf16 hi + lo parts, 64 x K in fragment order
  const uint16_t* lo;
  const uint16_t* Wb;   // the weights in B-operand order (bfrag_blocks of them)
  int nblk;             // 16-row blocks of Wb
  int seg_end[3];       // kDecStore: the bias segments' ends
  int K, N;             // K a multiple of 32; N output columns (kDecSwiglu: 2 F)
  int kc, ks;           // K per split (256 times 1-4, 6, 8, 12 or 16) and splits
  int cb;               // 16-column blocks per tile (dec_cb)
  int M;                // rows the epilogue writes (rows >= M are never stored)
  float* part;          // kDecParts: [ks, kMmaRows, N]; else [tiles, ks, 64 x 16 cb]
  int* ticket;          // [tiles] counters, zero between launches
  float* out;           // kDecStore: [M, ldo] written; kDecResidual: x [M, ldo] updated
  int ldo;
  const float* bias[3]; // kDecStore: per-segment bias or null
  uint16_t* ohi;        // kDecResidual: x * gain (64 x N); kDecSwiglu: 64 x F; fragment order
  uint16_t* olo;
  const float* gain;    // kDecResidual
  const float* ss_in;   // kDecStore / kDecSwiglu: [M, nss_in] sums of squares, or null
  int nss_in, hn;
  float eps;
  float* ss_out;        // kDecResidual: [M, N / kSsCols]
};

// 16-column blocks per tile: one for q/k/v and for residual GEMMs with K <=
// 2048 (more workgroups for the same split count, so fewer and smaller split
// tiles to merge, for activation rows short enough to read once per 16
// columns), four otherwise (SwiGLU: 32 gate + 32 up rows).  Measured on the
// 1.7B shape at 64 rows.
inline ATD_HD int dec_cb(int epi, int K) {
  return epi == kDecStore || (epi == kDecResidual && K <= 2048) ? 1 : 4;
}
inline ATD_HD int dec_tiles(int N, int epi, int K) {
  const int tc = 16 * dec_cb(epi, K);
  return epi == kDecSwiglu ? (N / 2 + tc / 2 - 1) / (tc / 2) : (N + tc - 1) / tc;
}

// K per split (kc) of a k_gemm_dec launch over `tiles` column tiles: as
// many splits as keep the launch within one workgroup per compute unit (all
// workgroups resident at once, so the last one of a tile never waits for a
// second round), at least one K step per wave and at most kDecMaxSteps; the
// steps per wave are rounded up to a count the kernel is built for.
inline int dec_kc(int tiles, int K) {
  const int span = kDecWaves * kDecKStep;   // K of one step of every wave
  const int nall = (K + span - 1) / span;   // steps of the whole K range
  int ks = kMmaCUs / tiles;
  if (ks < 1) ks = 1;
  if (ks > nall) ks = nall;
  int nks = (nall + ks - 1) / ks;
  if (nks < (nall + kDecMaxSteps - 1) / kDecMaxSteps) nks = (nall + kDecMaxSteps - 1) / kDecMaxSteps;
  nks = nks <= 4 ? nks : (nks <= 8 ? (nks + 1) / 2 * 2 : (nks + 3) / 4 * 4);
  if (nks > kDecMaxSteps) nks = kDecMaxSteps;
  return nks * span;
}

// RMSNorm(x) W^T = inv_m * ((x * g) W^T) with inv_m = 1 / sqrt(mean(x_m^2) + eps):
// the residual reduction leaves x * g (the next GEMM's input, as hi/lo) and
// partial sums of squares of x; the reduction after that GEMM applies inv_m.
struct ReduceArgs {
  const float* part;   // [ks, mrows, N]
  int ks, N, M;        // ks = 0: no partials (kRedResidual then only refreshes hi/lo, ss)
  int mrows;           // row stride of a split's partials
  const float* bias[3];  // kRedStore: per-segment bias or null
  int seg_end[3];
  float* out;          // kRedStore: [M, ldo] written; kRedResidual: [M, ldo] updated
  int ldo;
  uint16_t* hi;        // kRedResidual: x * gain; kRedSwiglu: the activation ([M, N or N/2])
  uint16_t* lo;
  const float* gain;   // kRedResidual: gain of the next norm; kRedStore: gain for y_out
  // kRedResidual writes ss [M, nss] (kSsCols-column partial sums of squares
  // of the updated rows); kRedStore / kRedSwiglu with ss set scale the sums by
  // inv_m from ss [M, nss] over hn columns.
  float* ss;
  int nss, hn;
  float eps;
  const float* x;      // kRedStore: rows whose norm goes to y_out ([M, hn])
  float* y_out;        // kRedStore: x * inv_m * gain [M, hn] or null
  int frag;            // hi / lo written in MFMA-fragment order (frag_off; M <= 64)
};

// ---------------------------------------------------------------- launchers
// Each returns the first HIP error of its launches (hipSuccess otherwise).
hipError_t launch_embed(const EmbedArgs& a, int bf16, hipStream_t s);
hipError_t launch_gemv(const GemvArgs& a, int epi, bool norm, int wtype, hipStream_t s);
// Rows of every weight matrix that block b of a launch_gemv of this shape
// reads (rows b * br .. b * br + br - 1), and the bytes of a dense weight row.
void gemv_block_rows(int N, int K, int wtype, int& br, size_t& row_bytes);

struct QuantArgs {
  const void* w;         // [rows, cols] float32 or bf16
  int bf16;
  int64_t rows;
  int cols;
  int q4;                // 0: int8 codes, 1: 4-bit pairs
  void* codes;
  uint16_t* scales;      // [rows, cols / kQBlock]
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);

// Codec convolutions as GEMMs over (input channel, tap): output frame t of
// phase p is y[co * ldy + t * ystride + p] = bias[co] + sum over r = ci*K + j
// of w[p][co][r] * x[ci][t - (K-1-j) * dil]  (x = 0 outside [0, T)).
struct ConvArgs {
  const float* x;      // [cin, T] channel-major
  const float* w;      // [P][cout][cin * K]
  const float* bias;   // [cout] or null
  float* y;
  int cin, cout, T, K, dil;
  int ldy, ystride, P;
  int accumulate;      // 1: y += the result (a residual add)
};
hipError_t launch_conv(const ConvArgs& a, hipStream_t s);
// [cin][cout][2s] transposed-convolution weights -> [s][cout][cin * 2] phases
// (tap 0 reads the previous frame with w[..][p + s], tap 1 the frame with w[..][p])
hipError_t launch_pack_transconv(const float* w, int cin, int cout, int s_, float* packed,
                                 hipStream_t s);
hipError_t launch_rope_append(const RopeArgs& a, int bf16, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int bf16, int D, int r, hipStream_t s);
// Causal attention of a prefill chunk (rows in kRowsPrefill mode, non-fused,
// k_direct set) in one pass over key tiles: writes o (or o_hi / o_lo).
hipError_t launch_attn_prefill(const AttnArgs& a, int bf16, int D, int r, hipStream_t s);
hipError_t launch_advance(const SlotTables& st, RowMap rows, int M, hipStream_t s);
// dst[i] = slots[i], i < n (host values, written on the stream)
hipError_t launch_slot_list(int32_t* dst, const int32_t* slots, int n, hipStream_t s);
// RoPE rows of a call with rotary positions pos3 [M][3] (t, h, w): row m,
// frequency i takes cos/sin of the position table at pos3[m][c(i)], c(i) = 1
// when i % 3 == 1 and i < 3 sec_h, 2 when i % 3 == 2 and i < 3 sec_w, else 0;
// positions clamped into [0, max_ctx).
hipError_t launch_mrope_rows(const int32_t* pos3, int M, int half, int sec_h, int sec_w,
                             int max_ctx, const float* cos_t, const float* sin_t, float* rcos,
                             float* rsin, hipStream_t s);
hipError_t launch_set_slot(const SlotTables& st, int slot, void* const* k, void* const* v,
                           int cap, int pos, int set_ptrs, hipStream_t s);
hipError_t launch_kv_copy(const KvCopyArgs& a, hipStream_t s);
hipError_t launch_argmax(const ArgmaxArgs& a, hipStream_t s);
// Allocation-free token choice: the argmax partials of greedy_argmax_noalloc
// live in a fixed device array of kNoAllocScratchFloats floats (one per GPU);
// its address on the current device (taken once per device) goes to *out.
constexpr size_t kNoAllocScratchFloats = size_t(1) << 16;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(float** out);
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);
hipError_t launch_record_token(const int32_t* tok, int32_t* out, int32_t* counter, hipStream_t s);
// out[*counter * n + i] = src[i] for i < n (out may be null), then ++*counter; n <= 64
hipError_t launch_record_tokens(const int32_t* src, int n, int32_t* out, int32_t* counter,
                                hipStream_t s);
// dst[i] = src[i], i < n
hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
// one full read of `bytes` (a multiple of 16) at buf, 16-byte loads
hipError_t launch_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// The same product over 128 x 128 output tiles (calls of more than one row
// tile: prefill chunks); same arguments and partials layout.
hipError_t launch_gemm_tile(const GemmArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, int epi, hipStream_t s);
hipError_t launch_gemm_dec(const DecGemmArgs& a, int epi, hipStream_t s);
hipError_t launch_swizzle_b(const SwizzleArgs& a, hipStream_t s);

}  // namespace atd
