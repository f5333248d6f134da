// HIP kernels of the decode step for gfx950 (CDNA4, wave64).
//
// The step of one layer follows the per-layer sequence profiled in the
// qwen3-tts-hip OPTIMIZATION_LOG (DecodeStepStack entry): input norm, q/k/v
// projection, q/k layout + cache write, attention, output projection +
// residual, post norm, gate/up projection, SwiGLU, down projection +
// residual.  Here it is five launches: the norms are fused into the
// projection that consumes them, SwiGLU into the gate/up projection, the
// residual adds into the projections that produce them, the QK norm, RoPE
// and cache append into the attention, and no layout permute exists (the
// cache row is written in its final [Hkv, S, D] place).
//
// At batch 1 the step is bound by HBM bandwidth and launch latency: every
// weight byte is read once and used for one multiply-add, so the projections
// are GEMVs (k_gemv) that stream 16-byte vectors of weights per lane, all 64
// lanes of a wave on consecutive addresses of a row, with the input row held
// in registers.  The attention launch also carries workgroups that load the
// next launches' weights into the L2 of the XCDs that will read them
// (l2_prefetch), and weights read once are streamed with the nontemporal
// cache policy so that they do not evict those lines.  From 5 rows on, the projections run on the matrix cores:
// k_gemm_dec for chunks of up to 64 rows (split reduction and epilogue in
// the same launch), k_gemm_tile / k_gemm for prefill chunks, with the
// float32 activations as bf16 hi + lo operands.
//
// Attention at decode reads the K and V rows once; each row's key range is
// split into chunks set by its valid length (split-K over the sequence)
// whose partial softmax states (running max, sum, weighted V) are merged in a
// fixed order, inside the launch for up to 4 rows and by a second launch
// (k_attn_merge) for more, so results depend neither on the cache capacity
// nor on launch timing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

namespace atd {

// ------------------------------------------------------------------ helpers

// Cross-lane moves through DPP (no LDS traffic).  Controls: quad_perm
// [1,0,3,2] = xor 1, quad_perm [2,3,0,1] = xor 2, row_half_mirror pairs lane
// i with 7-i of its 8-lane half row, row_mirror pairs i with 15-i of its
// 16-lane row, row_ror:8 rotates a row by 8 lanes (= xor 8).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppRor8 = 0x128;

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32, 64), result in
// every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Inclusive prefix sum over the wave by DPP: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the last lane of rows 0 / 2 added into rows 1 / 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).  Lanes
// without a source (or masked off) add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_rows<0x111, 0xF>(v);
  v += dpp_rows<0x112, 0xF>(v);
  v += dpp_rows<0x114, 0xF>(v);
  v += dpp_rows<0x118, 0xF>(v);
  v += dpp_rows<0x142, 0xA>(v);
  v += dpp_rows<0x143, 0xC>(v);
  return v;
}

// Wave-wide sum, identical in every lane: rows of 16 by DPP, then the four
// row sums read out and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even
  return (uint16_t)(u >> 16);
}

template <typename T>
struct Vec16;  // 16-byte vector of T, unpacked to float
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};
template <>
struct Vec16<uint16_t> {  // bf16 bit patterns
  static constexpr int N = 8;
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xffff0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xffff0000u);
    f[4] = __uint_as_float(r.z << 16);
    f[5] = __uint_as_float(r.z & 0xffff0000u);
    f[6] = __uint_as_float(r.w << 16);
    f[7] = __uint_as_float(r.w & 0xffff0000u);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte load through the global address space (pointers taken from memory
// are generic; a flat load would also count against the scalar-memory
// counter and couple to unrelated scalar waits).
typedef unsigned int V4U32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(1))) const V4U32 GV4U32;
  const V4U32 v = *(GV4U32*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

// 8- and 2-byte loads through the global address space.
typedef unsigned int V2U32 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldg8(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(1))) const V2U32 GV2U32;
  const V2U32 v = *(GV2U32*)(p);
  return make_uint2(v.x, v.y);
#else
  return *reinterpret_cast<const uint2*>(p);
#endif
}
__device__ __forceinline__ uint32_t ldg4(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(__attribute__((address_space(1))) const uint32_t*)(p);
#else
  return *reinterpret_cast<const uint32_t*>(p);
#endif
}

// The 16-byte load with the nontemporal cache policy (bit nt), for weights
// that a launch streams once: the caches let such lines go first, so the
// stream does not push out what is read again (activations, weights
// prefetched into L2 for the next launch).
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(1))) const V4U32 GV4U32;
  const V4U32 v = __builtin_nontemporal_load((GV4U32*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}
__device__ __forceinline__ uint16_t ldg2(const uint16_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(__attribute__((address_space(1))) const uint16_t*)(p);
#else
  return *p;
#endif
}

// IEEE fp16 bit patterns <-> float (conversion rounds to nearest even).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Weight chunks of the GEMV: one load per lane per row and chunk, unpacked to
// N floats.  Quantized formats unpack to code + OFF (unsigned, so each byte
// converts in one instruction) and carry one fp16 scale per kQBlock weights;
// the offset leaves once per chunk through the chunk's input sum.  Their
// chunks are smaller than 16 bytes so that a matrix spreads over as many
// waves as a bf16 one of the same shape.
struct WQ8 {};   // int8 codes
struct WQ4 {};   // 4-bit codes + 8: weight 2i in the low nibble of byte i, 2i+1 high

// bytes of a quantized chunk (one load per lane per row): 16 weights either
// way, so K / N <= 512 chunks and at most 4 per lane (measured: 8-byte int8
// or 4-byte 4-bit chunks run no faster; 16-byte 4-bit chunks halve the lanes
// a row spreads over and run 2x slower)
constexpr int kQ8ChunkBytes = 16;
constexpr int kQ4ChunkBytes = 8;

template <int BYTES>
__device__ __forceinline__ uint4 ldg_chunk(const char* p) {
  if constexpr (BYTES == 16) {
    return ldg16(p);
  } else if constexpr (BYTES == 8) {
    const uint2 v = ldg8(p);
    return make_uint4(v.x, v.y, 0u, 0u);
  } else {
    static_assert(BYTES == 4, "4, 8 or 16-byte chunks");
    return make_uint4(ldg4(p), 0u, 0u, 0u);
  }
}

template <typename WT>
struct WFmt {    // dense float32 / bf16
  static constexpr int N = Vec16<WT>::N, BYTES = 16;
  static constexpr bool Q = false;
  static constexpr float OFF = 0.f;
  __device__ static __forceinline__ uint4 load(const char* p) { return ldg16(p); }
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) { Vec16<WT>::unpack(r, f); }
};
// bf16 weights loaded with the nontemporal policy: for decoders whose weights
// do not fit the memory-side cache (measured: the 1.7B step and the stand-alone
// gate/up GEMV faster; a decoder that fits, such as the ASR shape, slower)
struct Bf16Nt {};
template <>
struct WFmt<Bf16Nt> {
  static constexpr int N = 8, BYTES = 16;
  static constexpr bool Q = false;
  static constexpr float OFF = 0.f;
  __device__ static __forceinline__ uint4 load(const char* p) { return ldg16_nt(p); }
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) { Vec16<uint16_t>::unpack(r, f); }
};
template <>
struct WFmt<WQ8> {
  static constexpr int BYTES = kQ8ChunkBytes, N = BYTES;
  static constexpr bool Q = true;
  static constexpr float OFF = 128.f;
  __device__ static __forceinline__ uint4 load(const char* p) { return ldg_chunk<BYTES>(p); }
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < BYTES / 4; ++j) {
      const uint32_t u = w[j] ^ 0x80808080u;   // code + 128 in every byte
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * j + b] = (float)((u >> (8 * b)) & 0xffu);
    }
  }
};
template <>
struct WFmt<WQ4> {
  static constexpr int BYTES = kQ4ChunkBytes, N = 2 * BYTES;
  static constexpr bool Q = true;
  static constexpr float OFF = 8.f;
  __device__ static __forceinline__ uint4 load(const char* p) { return ldg_chunk<BYTES>(p); }
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < BYTES / 4; ++j) {
      const uint32_t lo = w[j] & 0x0f0f0f0fu, hi = (w[j] >> 4) & 0x0f0f0f0fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f[8 * j + 2 * b] = (float)((lo >> (8 * b)) & 0xffu);
        f[8 * j + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xffu);
      }
    }
  }
};

__device__ __forceinline__ void row_of(const RowMap& r, const SlotTables& st, int m,
                                       int& slot, int& pos) {
  if (r.mode == kRowsPrefill) {
    slot = r.slot0;
    pos = r.row0 + m;
  } else {
    slot = step_slot(r, r.row0 + m);
    pos = st.pos[slot];
  }
}

// ------------------------------------------------------------------ embed
// x[m] = sum_g table_g[tok[m, g]] + extra[m]   (tables summed in order g)
template <typename T>
__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
  const int m = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.h) return;
  float s = 0.f;
  for (int g = 0; g < a.G; ++g) {
    int t = a.tok[m * a.G + g];
    t = t < 0 ? 0 : (t >= a.vocab[g] ? a.vocab[g] - 1 : t);
    const T* row = reinterpret_cast<const T*>(a.tab[g]) + (size_t)t * a.h;
    if constexpr (sizeof(T) == 2)
      s += __uint_as_float((uint32_t)row[i] << 16);
    else
      s += row[i];
  }
  if (a.extra) {
    const float* ex = a.extra + (a.extra_row ? (size_t)(*a.extra_row) * a.h : 0);
    s += ex[(size_t)m * a.h + i];
  }
  a.out[(size_t)m * a.h + i] = s;
}

// ------------------------------------------------------------------ QK norm + RoPE + append
// One (row m, head slot hh) of the raw projection: hh < Hq is a query head,
// then Hkv key heads, then Hkv value heads.  q and k heads get the optional
// per-head RMSNorm over D and rotate-half RoPE at the row's position; q goes
// to q_out, k and v are stored (rounded for a bf16 cache) into the cache row.
// All (row, head slot) items of a call: G = 64 / (D/2)
// items per wave, lane l of an item holding channels l and l + D/2 (the
// rotate-half pair, so the rotation needs no exchange); the QK-norm's sum of
// squares is a shuffle reduction over the item's lanes.  One wave per item
// (two at D = 64), no LDS or barriers (a prefill chunk has M x (Hq + 2 Hkv)
// items; at 512 rows of the 1.7B shape this form takes 6-7 us per layer,
// one 128-thread block per item with LDS reductions took 11 us).
template <typename KT, int D>
__global__ __launch_bounds__(256) void k_rope_append(RopeArgs a) {
  constexpr int half = D / 2, G = 64 / half;
  const int lane = threadIdx.x & 63, sub = lane / half, l = lane % half;
  const int nh = a.Hq + 2 * a.Hkv;
  const int item = (blockIdx.x * 4 + (threadIdx.x >> 6)) * G + sub;
  if (item >= a.M * nh) return;   // whole items only: the reduction stays within one
  const int m = item / nh, hh = item % nh;
  int slot, pos;
  row_of(a.rows, a.st, m, slot, pos);
  const int ld = nh * D;
  const int kind = hh < a.Hq ? 0 : (hh < a.Hq + a.Hkv ? 1 : 2);
  const int hd = kind == 0 ? hh : (kind == 1 ? hh - a.Hq : hh - a.Hq - a.Hkv);
  const int col = (kind == 0 ? 0 : (kind == 1 ? a.Hq * D : (a.Hq + a.Hkv) * D)) + hd * D;
  const float* src = a.qkv + (size_t)m * ld + col;
  float v0 = src[l], v1 = src[l + half];
  if (kind < 2) {
    if (a.qk_norm) {
      float s2 = v0 * v0 + v1 * v1;
#pragma unroll
      for (int off = 1; off < half; off <<= 1) s2 += __shfl_xor(s2, off, 64);
      const float inv = 1.0f / sqrtf(s2 / (float)D + a.eps);
      const float* g = kind == 0 ? a.q_norm : a.k_norm;
      v0 = v0 * inv * g[l];
      v1 = v1 * inv * g[l + half];
    }
    const size_t rr = (size_t)(a.rows.rope_rows ? a.rows.row0 + m : pos) * half;
    const float c = a.cos_t[rr + l], sn = a.sin_t[rr + l];
    const float x0 = v0, x1 = v1;
    v0 = x0 * c - x1 * sn;
    v1 = x1 * c + x0 * sn;
  }
  if (kind == 0) {
    float* q = a.q_out + ((size_t)m * a.Hq + hd) * D;
    q[l] = v0;
    q[l + half] = v1;
  } else {
    void* const* kv = a.st.kv + ((size_t)slot * a.st.L + a.layer) * 2;
    const int cap = a.st.cap[slot];
    KT* dst = reinterpret_cast<KT*>(kv[kind - 1]) + ((size_t)hd * cap + pos) * D;
    if constexpr (sizeof(KT) == 2) {
      dst[l] = f32_to_bf16(v0);
      dst[l + half] = f32_to_bf16(v1);
    } else {
      dst[l] = v0;
      dst[l + half] = v1;
    }
  }
}

// ------------------------------------------------------------------ GEMV
// out[m, n] = epi( sum_k W[n, k] * xin[m, k] ),  xin = x or RMSNorm(x) * gain
//
// A block of 4 waves owns (4 / KS) * RW consecutive output rows: 4 / KS
// groups of KS waves, each group RW rows whose K dimension is cut into KS
// slices (wave q takes slice q % KS of its group's rows).  RW = KS, or 4 for
// tall matrices with a short K (the ASR LM head), so that a wave's weight
// stream outweighs its input loads.  Every lane streams KI
// 16-byte chunks per row, so all 64 lanes of a wave read consecutive
// addresses of a row and a whole slice is in flight at once.  Load order
// follows the in-order memory counter: first the small operands the math
// needs early (the lane's slice of the input rows and the gain, and the
// epilogue's bias or residual), then the weights, so the norm's sum of
// squares and its cross-wave reduction run while the weights stream in.
// Partial dots of the KS slices meet in LDS and are added in a fixed order.
// MR input rows share every weight load.  Argument arrays are only indexed
// with constants (a run-time index would turn into a memory load of the
// argument block ahead of everything else).
template <typename T>
__device__ __forceinline__ T pick3(const T (&v)[3], int i) {
  return i == 0 ? v[0] : (i == 1 ? v[1] : v[2]);
}

template <typename WT, int MR, int KS, int KI, int EPI, bool NORM, int RW>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  using F = WFmt<WT>;
  constexpr int VEC = F::N;
  constexpr int NW = EPI == kEpiSwiglu ? 2 : 1;
  constexpr int BR = (4 / KS) * RW;   // rows per block
  __shared__ float red_ss[4][MR];
  __shared__ float red_acc[4][RW][MR][NW];
  const int tid = threadIdx.x, lane = tid & 63, q = tid >> 6;
  const int ks = q % KS, grp = q / KS;
  const int K = a.K, nk = K / VEC, ql = (nk + KS - 1) / KS;  // last slice may be short
  const int row0 = blockIdx.x * BR + grp * RW;
  const bool active = row0 < a.N;

  // 1) small operands: input slice, gain slice, epilogue operand
  float xv[MR][KI][VEC];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int cq = lane + 64 * i;
      const int c = ks * ql + cq;
      const bool in = cq < ql && c < nk;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const uint4 t = in ? ldg16(a.x + (size_t)m * a.ldx + (size_t)c * VEC + e) : make_uint4(0, 0, 0, 0);
        xv[m][i][e] = __uint_as_float(t.x);
        xv[m][i][e + 1] = __uint_as_float(t.y);
        xv[m][i][e + 2] = __uint_as_float(t.z);
        xv[m][i][e + 3] = __uint_as_float(t.w);
      }
    }
  float gv[KI][VEC];
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int cq = lane + 64 * i;
      const int c = ks * ql + cq;
      const bool in = cq < ql && c < nk;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const uint4 t = in ? ldg16(a.gain + (size_t)c * VEC + e) : make_uint4(0, 0, 0, 0);
        gv[i][e] = __uint_as_float(t.x);
        gv[i][e + 1] = __uint_as_float(t.y);
        gv[i][e + 2] = __uint_as_float(t.z);
        gv[i][e + 3] = __uint_as_float(t.w);
      }
    }
  }
  // thread (m, rr) of the first BR*MR threads finishes output row rr of input m
  const int em = tid / BR, err = tid % BR, erow = blockIdx.x * BR + err;
  const bool fin = tid < BR * MR && erow < a.N;
  float eo = 0.f;
  if (fin) {
    if constexpr (EPI == kEpiStore) {
      const int gs = erow < a.seg_end[0] ? 0 : (erow < a.seg_end[1] ? 1 : 2);
      const float* b = pick3(a.bias, gs);
      const int gbeg = gs == 0 ? 0 : (gs == 1 ? a.seg_end[0] : a.seg_end[1]);
      if (b) eo = b[erow - gbeg];
    } else if constexpr (EPI == kEpiResidual) {
      eo = a.out[(size_t)em * a.ldo + erow];
    }
  }

  // 2) weights: every lane issues all its loads (addresses clamped into the
  // matrix; positions past the slice meet zero inputs and rows past N are
  // never stored), so the number of loads behind the small operands is fixed
  // and waiting for those does not wait for the weights
  const int rowc = active ? row0 : a.N - 1;
  const int sg = rowc < a.seg_end[0] ? 0 : (rowc < a.seg_end[1] ? 1 : 2);
  const int sbeg = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
  const int nr = min(RW, pick3(a.seg_end, sg) - rowc);   // >= 1
  const size_t rowb = (size_t)nk * F::BYTES;   // bytes of a weight row
  const char* Wp = reinterpret_cast<const char*>(pick3(a.W, sg)) + (size_t)(rowc - sbeg) * rowb;
  const char* W2p =
      EPI == kEpiSwiglu ? reinterpret_cast<const char*>(a.W2) + (size_t)rowc * rowb : nullptr;
  const int nb = K / kQBlock;   // scale blocks per row (quantized types)
  const uint16_t* Sp = F::Q ? pick3(a.S, sg) + (size_t)(rowc - sbeg) * nb : nullptr;
  const uint16_t* S2p = F::Q && EPI == kEpiSwiglu ? a.S2 + (size_t)rowc * nb : nullptr;
  uint4 w[KI][RW][NW];
  uint16_t sc[KI][RW][NW];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int cq = lane + 64 * i;
    const int c = min(ks * ql + cq, nk - 1);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const size_t rr = (size_t)min(r, nr - 1);
      const size_t off = rr * rowb + (size_t)c * F::BYTES;
      w[i][r][0] = F::load(Wp + off);
      if constexpr (NW == 2) w[i][r][1] = F::load(W2p + off);
      if constexpr (F::Q) {
        const size_t so = rr * nb + (size_t)c * VEC / kQBlock;
        sc[i][r][0] = ldg2(Sp + so);
        if constexpr (NW == 2) sc[i][r][1] = ldg2(S2p + so);
      }
    }
  }
  // keep the scheduler from hoisting the norm (which waits for the small
  // operands) between the weight loads
  __builtin_amdgcn_sched_barrier(0);

  // 3) the norm, while the weights arrive
  if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < KI; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += xv[m][i][e] * xv[m][i][e];
      const float v = wave_sum(ss);
      if (lane == 0) red_ss[q][m] = v;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float tot = 0.f;
#pragma unroll
      for (int j = 0; j < KS; ++j) tot += red_ss[grp * KS + j][m];
      const float inv = 1.0f / sqrtf(tot / (float)K + a.eps);
#pragma unroll
      for (int i = 0; i < KI; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) xv[m][i][e] = xv[m][i][e] * inv * gv[i][e];
      if (a.y_out && blockIdx.x == 0 && grp == 0) {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const int cq = lane + 64 * i;
          const int c = ks * ql + cq;
          if (cq < ql && c < nk) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
              *reinterpret_cast<float4*>(a.y_out + (size_t)m * K + (size_t)c * VEC + e) =
                  make_float4(xv[m][i][e], xv[m][i][e + 1], xv[m][i][e + 2], xv[m][i][e + 3]);
          }
        }
      }
    }
  }

  // 4) dot products (quantized: per chunk, scale * (sum (code + OFF) x - OFF sum x))
  float xs[MR][KI];
  if constexpr (F::Q) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t += xv[m][i][e];
        xs[m][i] = t;
      }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          float wf[VEC];
          F::unpack(w[i][r][t], wf);
          if constexpr (F::Q) {
            float dq = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) dq = fmaf(wf[e], xv[m][i][e], dq);
            acc = fmaf(f16_bits_to_f32(sc[i][r][t]), fmaf(-F::OFF, xs[m][i], dq), acc);
          } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc = fmaf(wf[e], xv[m][i][e], acc);
          }
        }
        acc = wave_sum(acc);
        if (lane == 0) red_acc[q][r][m][t] = acc;
      }
  __syncthreads();
  if (fin) {
    const int g = err / RW, r = err % RW;
    float v[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < KS; ++j) acc += red_acc[g * KS + j][r][em][t];
      v[t] = acc;
    }
    float* o = a.out + (size_t)em * a.ldo + erow;
    if constexpr (EPI == kEpiSwiglu)
      *o = v[0] / (1.0f + expf(-v[0])) * v[NW - 1];
    else
      *o = eo + v[0];
  }
}

// ------------------------------------------------------------------ block quantization
// One thread per block of kQBlock weights of a row: d = max|w| / QMAX,
// code = w / d rounded half away from zero (float32), scale = fp16(d).
template <typename WT, bool Q4>
__global__ __launch_bounds__(256) void k_quantize(QuantArgs a) {
  const int nb = a.cols / kQBlock;
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= a.rows * nb) return;
  const int64_t row = blk / nb;
  const int b = (int)(blk - row * nb);
  constexpr int VN = Vec16<WT>::N;
  const char* src = reinterpret_cast<const char*>(a.w) +
                    ((size_t)row * a.cols + (size_t)b * kQBlock) * sizeof(WT);
  float v[kQBlock];
#pragma unroll
  for (int c = 0; c < kQBlock / VN; ++c) Vec16<WT>::unpack(ldg16(src + 16 * c), v + c * VN);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < kQBlock; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const float qmax = Q4 ? 7.f : 127.f;
  const float d = amax / qmax;
  int q[kQBlock];
#pragma unroll
  for (int e = 0; e < kQBlock; ++e) {
    float t = d > 0.f ? roundf(v[e] / d) : 0.f;
    t = fminf(fmaxf(t, -qmax), qmax);
    q[e] = (int)t;
  }
  a.scales[(size_t)row * nb + b] = f32_to_f16_bits(d);
  if constexpr (Q4) {
    uint32_t wds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t wd = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = 8 * j + 2 * t;
        wd |= ((uint32_t)(q[e] + 8) | ((uint32_t)(q[e + 1] + 8) << 4)) << (8 * t);
      }
      wds[j] = wd;
    }
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.codes) +
                                          (size_t)row * (a.cols / 2) + (size_t)b * (kQBlock / 2));
    *dst = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  } else {
    uint32_t wds[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t wd = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) wd |= ((uint32_t)q[4 * j + t] & 0xffu) << (8 * t);
      wds[j] = wd;
    }
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.codes) +
                                          (size_t)row * a.cols + (size_t)b * kQBlock);
    dst[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    dst[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
  }
}

// ------------------------------------------------------------------ codec convolutions
// (k_conv1d follows the matrix-core GEMM section below: it shares its types)

__global__ __launch_bounds__(256) void k_pack_transconv(const float* w, int cin, int cout, int s_,
                                                        float* packed) {
  const size_t n = (size_t)s_ * cout * cin * 2;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int j = (int)(i & 1);
    const size_t q = i >> 1;
    const int ci = (int)(q % cin);
    const size_t q2 = q / cin;
    const int co = (int)(q2 % cout), p = (int)(q2 / cout);
    const int k = j == 0 ? p + s_ : p;   // tap 0: previous frame, tap 1: this frame
    packed[i] = w[((size_t)ci * cout + co) * (2 * s_) + k];
  }
}

// ------------------------------------------------------------------ attention
// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi): ~16 significant bits
// in two bf16 matrix-core operands
__device__ __forceinline__ void split_hi_lo(float v, uint16_t& h, uint16_t& l) {
  h = f32_to_bf16(v);
  l = f32_to_bf16(v - __uint_as_float((uint32_t)h << 16));
}

// Split-K decode attention, one split per wave.  Block (split group, kv head
// g, row m); wave w takes split 4*blockIdx.x + w of the row's key range
// (attn_chunk keys each, from its valid length) for the R query heads that
// share KV head g.  A key row of D elements is read by LPK lanes with
// 16-byte loads, so a wave covers KPW keys per load; U key groups are in
// flight per iteration.  Each lane group keeps an online softmax state
// (max, sum, weighted V); groups are merged with shuffles in a fixed order,
// then the block's four waves through LDS in wave order.  A (row, KV head)
// with one block writes o there; with several, each block writes its state
// at the device-coherent level and takes a ticket, and the last block to
// arrive merges all of them in block order, so the result never depends on
// the order of arrival (and the combine needs no launch of its own).
//
// Fused mode (decode steps): the wave applies the QK norm and RoPE to its raw
// queries itself, and the wave of the row's last split builds the new k/v
// row (norm, RoPE, rounding to the cache dtype), stores it at the row's
// position and uses those register values for that key.  Only that wave
// touches the new row, so no other synchronisation is needed.

template <typename KT, int VEC>
__device__ __forceinline__ uint4 pack_kv(const float (&v)[VEC]) {
  uint4 r;
  if constexpr (sizeof(KT) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    r = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    r = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                   __float_as_uint(v[3]));
  }
  return r;
}

// Attention output of 4 channels at o[off] (or their bf16 hi / lo parts).
template <int D>
__device__ __forceinline__ void store_o4(const AttnArgs& a, size_t off, float4 v) {
  if (a.o_hi) {
    const float f[4] = {v.x, v.y, v.z, v.w};
    uint16_t hv[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_hi_lo(f[i], hv[i], lv[i]);
    if (a.o_frag) {   // off = m * Hq * D + column, the column a multiple of 4
      const int HD = a.Hq * D;
      off = frag_off((int)(off / HD), (int)(off % HD));
    }
    *reinterpret_cast<uint2*>(a.o_hi + off) =
        make_uint2(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16));
    *reinterpret_cast<uint2*>(a.o_lo + off) =
        make_uint2(lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16));
  } else {
    *reinterpret_cast<float4*>(a.o + off) = v;
  }
}

// Stores and loads at the device-coherent level (relaxed atomics of device
// scope: they bypass the per-XCD caches), for values one workgroup writes
// and another, possibly on another XCD, reads within the same kernel.
__device__ __forceinline__ uint64_t pack2(float x, float y) {
  return (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
}
__device__ __forceinline__ void store_coherent2(float* p, float x, float y) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), pack2(x, y), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent4(float* p, float4 v) {
  store_coherent2(p, v.x, v.y);
  store_coherent2(p + 2, v.z, v.w);
}
__device__ __forceinline__ void load_coherent2(const float* p, float& x, float& y) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  x = __uint_as_float((uint32_t)u);
  y = __uint_as_float((uint32_t)(u >> 32));
}
__device__ __forceinline__ float4 load_coherent4(const float* p) {
  float4 v;
  load_coherent2(p, v.x, v.y);
  load_coherent2(p + 2, v.z, v.w);
  return v;
}

// Prefetch workgroup j of P in a launch whose workgroup `lin` it is (on XCD
// lin % 8): with the other prefetch workgroups of its XCD it loads every
// 16-byte chunk that the covered blocks b = x, x + 8, ... of each region
// read.  256 threads, eight loads in flight per thread: a share arrives over
// a few round trips, which keeps the prefetch from crowding out the loads of
// the launch's own workgroups (a whole share in one round trip was slower).
__device__ __forceinline__ void l2_prefetch(const L2Prefetch& p, int j, int P, int lin) {
  constexpr int NT = 256, U = 8;
  const int x = lin & 7;
  const int j0 = (x - (lin - j)) & 7;               // first prefetch workgroup on XCD x
  const int per = (P - j0 + 7) >> 3, idx = j >> 3;  // workgroups on XCD x, this one's index
  uint32_t acc = 0;
  for (int r = 0; r < p.nreg; ++r) {
    const uint32_t c16 = (uint32_t)(p.bb[r] >> 4);
    const int nb = (p.nblk[r] - x + 7) >> 3;   // covered blocks on XCD x
    if (nb <= 0) continue;
    const uint32_t total = (uint32_t)nb * c16;
    for (uint32_t t0 = (uint32_t)idx * NT * U + threadIdx.x; t0 < total; t0 += (uint32_t)per * NT * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t t = t0 + u * NT;
        const uint32_t b = (uint32_t)x + 8u * (t / c16), c = t % c16;
        v[u] = t < total ? ldg16(p.base[r] + (size_t)b * p.bb[r] + (size_t)c * 16)
                         : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc |= v[u].x | v[u].y | v[u].z | v[u].w;
    }
  }
  asm volatile("" ::"v"(acc));   // the loads count as used
}

// Merge of the partial states of the nblk blocks of (row m, KV head g) in
// block order, by the 256 threads of one workgroup: P phases per (query head,
// channel group) item, phase p merging blocks p, p + P, ... online, then the
// phases merged in order; writes the attention output.  COH: read the states
// at the device-coherent level (written in the same launch), else plainly
// (written by an earlier launch).
template <int D, int R, bool COH>
__device__ __forceinline__ void attn_merge_states(const AttnArgs& a, int m, int g, int nblk) {
  constexpr int NC = D / 4;
  constexpr int ITEMS = R * NC;
  constexpr int P = 256 / ITEMS;
  __shared__ float s_pm[P][ITEMS], s_pl[P][ITEMS];
  __shared__ float4 s_pa[P][ITEMS];
  const int tid = threadIdx.x;
  const int item = tid % ITEMS, j = item / NC, c = item % NC;
  const size_t head = (size_t)m * a.Hq + g * R + j;
  const int ph = tid / ITEMS;
  if (ph < P) {
    float M = -1e30f, L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    // a batch of partials is loaded together (one memory round trip), then
    // merged in order; indexes past the last block re-read it and are skipped
    constexpr int NB = 8;
    for (int b0 = ph; b0 < nblk; b0 += NB * P) {
      float bm[NB], bl[NB];
      float4 v[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const size_t pb = head * a.nsplit_max + min(b0 + i * P, nblk - 1);
        if constexpr (COH) {
          load_coherent2(a.pml + pb * 2, bm[i], bl[i]);
          v[i] = load_coherent4(a.pacc + pb * D + 4 * c);
        } else {
          const float2 t = *reinterpret_cast<const float2*>(a.pml + pb * 2);
          bm[i] = t.x;
          bl[i] = t.y;
          v[i] = *reinterpret_cast<const float4*>(a.pacc + pb * D + 4 * c);
        }
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (b0 + i * P < nblk) {
          const float nm = fmaxf(M, bm[i]);
          const float ca = expf(M - nm), cb = expf(bm[i] - nm);
          L = L * ca + bl[i] * cb;
          A = make_float4(A.x * ca + v[i].x * cb, A.y * ca + v[i].y * cb,
                          A.z * ca + v[i].z * cb, A.w * ca + v[i].w * cb);
          M = nm;
        }
      }
    }
    s_pm[ph][item] = M;
    s_pl[ph][item] = L;
    s_pa[ph][item] = A;
  }
  __syncthreads();
  if (tid < ITEMS) {
    float M = s_pm[0][item];
#pragma unroll
    for (int q = 1; q < P; ++q) M = fmaxf(M, s_pm[q][item]);
    float L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const float cq = expf(s_pm[q][item] - M);
      L = fmaf(s_pl[q][item], cq, L);
      const float4 v = s_pa[q][item];
      A = make_float4(fmaf(v.x, cq, A.x), fmaf(v.y, cq, A.y), fmaf(v.z, cq, A.z), fmaf(v.w, cq, A.w));
    }
    store_o4<D>(a, head * D + 4 * c, make_float4(A.x / L, A.y / L, A.z / L, A.w / L));
  }
}

// DEFER: the blocks of a (row, KV head) only write their partial states;
// k_attn_merge (the next launch) merges them.  Otherwise the last block to
// arrive merges them in this launch.
template <typename KT, int D, int R, int LPK, int U, bool DEFER>
__global__ __launch_bounds__(256) void k_attn_split(AttnArgs a) {
  constexpr int VEC = Vec16<KT>::N;   // channels per 16-byte load
  constexpr int DPL = D / LPK;        // channels per lane (LPK lanes per key row)
  constexpr int NV = DPL / VEC;       // 16-byte loads per lane per row
  constexpr int KPW = 64 / LPK;       // key rows per wave-wide load
  constexpr int TILE = KPW * U;       // keys per wave per tile (U rows per lane group)
  static_assert(NV >= 1 && DPL % 4 == 0, "a lane holds whole 16-byte groups");

  if ((int)blockIdx.z == a.M) {   // the prefetch slice
    const int j = blockIdx.x + gridDim.x * blockIdx.y, P = gridDim.x * gridDim.y;
    l2_prefetch(a.pf, j, P, j + P * a.M);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x * 4 + wave, g = blockIdx.y, m = blockIdx.z;
  const int sub = lane / LPK, dl = (lane % LPK) * DPL;
  const int ldq = (a.Hq + 2 * a.Hkv) * D;
  // the raw query rows do not depend on the position: load them with it
  float qv[R][DPL];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int h = g * R + j;
    const float* qp = a.fused ? a.qkv + (size_t)m * ldq + (size_t)h * D + dl
                              : a.q + ((size_t)m * a.Hq + h) * D + dl;
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
      const float4 t = *reinterpret_cast<const float4*>(qp + e);
      qv[j][e] = t.x;
      qv[j][e + 1] = t.y;
      qv[j][e + 2] = t.z;
      qv[j][e + 3] = t.w;
    }
  }
  int slot, pos;
  row_of(a.rows, a.st, m, slot, pos);
  const int len = pos + 1;
  const int chunk = attn_chunk(len, a.M, a.Hkv, a.waves);
  const int k0 = split * chunk;
  // a block whose four splits all start past the row's length has nothing to
  // do (uniform over the block); a wave of a live block whose split does
  // still takes part in the block's merge, with an empty state
  if (blockIdx.x * 4 * chunk >= len) return;
  if (a.nsplit_max == 1 && k0 >= len) return;   // single split: no merge below
  const bool has_keys = k0 < len;
  const int k1 = min(len, k0 + chunk);
  const bool owns_new = a.fused && has_keys && k1 == len;
  // the cached keys this wave reads: the owner of the new row takes that row
  // from its registers, first, and reads the cache only below it
  const int kend = owns_new ? k1 - 1 : k1;

  // position-dependent small loads first (RoPE table, gains, the new row),
  // then the cache rows: the in-order memory counter lets the query math
  // start before the rows arrive
  const int half = D / 2;
  const size_t rr = (size_t)(a.rows.rope_rows ? a.rows.row0 + m : pos) * half;
  const float* cp = a.cos_t + rr + (dl % half);
  const float* sp = a.sin_t + rr + (dl % half);
  float4 cs[DPL / 4], sn[DPL / 4];
  if (a.fused) {
#pragma unroll
    for (int e = 0; e < DPL / 4; ++e) {
      cs[e] = *reinterpret_cast<const float4*>(cp + 4 * e);
      sn[e] = *reinterpret_cast<const float4*>(sp + 4 * e);
    }
  }
  float kf[DPL], vf[DPL];
  if (owns_new) {
    const float* kp = a.qkv + (size_t)m * ldq + (size_t)(a.Hq + g) * D + dl;
    const float* vp = a.qkv + (size_t)m * ldq + (size_t)(a.Hq + a.Hkv + g) * D + dl;
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
      const float4 tk = *reinterpret_cast<const float4*>(kp + e);
      const float4 tv = *reinterpret_cast<const float4*>(vp + e);
      kf[e] = tk.x; kf[e + 1] = tk.y; kf[e + 2] = tk.z; kf[e + 3] = tk.w;
      vf[e] = tv.x; vf[e + 1] = tv.y; vf[e + 2] = tv.z; vf[e + 3] = tv.w;
    }
  }

  int cap;
  const KT *Kh, *Vh;
  if (a.k_direct) {
    cap = a.cap_direct;
    Kh = reinterpret_cast<const KT*>(a.k_direct);
    Vh = reinterpret_cast<const KT*>(a.v_direct);
  } else {
    cap = a.st.cap[slot];
    void* const* kvp = a.st.kv + ((size_t)slot * a.st.L + a.layer) * 2;
    Kh = reinterpret_cast<const KT*>(kvp[0]);
    Vh = reinterpret_cast<const KT*>(kvp[1]);
  }
  Kh += (size_t)g * cap * D + dl;
  Vh += (size_t)g * cap * D + dl;

  // the QK-norm gains of the lane's channels, also ahead of the cache rows
  float4 gq[DPL / 4], gk[DPL / 4];
  if (a.fused && a.qk_norm) {
#pragma unroll
    for (int e = 0; e < DPL / 4; ++e) gq[e] = *reinterpret_cast<const float4*>(a.q_norm + dl + 4 * e);
    if (owns_new) {
#pragma unroll
      for (int e = 0; e < DPL / 4; ++e) gk[e] = *reinterpret_cast<const float4*>(a.k_norm + dl + 4 * e);
    }
  }

  // keys past the range end are clamped to its last key (always in bounds;
  // row 0 when the range is empty, then never used) and masked out in the
  // softmax
  uint4 kr[U][NV], vr[U][NV];
  const int klast = kend > 0 ? kend - 1 : 0;
  auto load = [&](int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(kb + u * KPW + sub, klast);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        kr[u][v] = ldg16(Kh + (size_t)key * D + v * VEC);
        vr[u][v] = ldg16(Vh + (size_t)key * D + v * VEC);
      }
    }
  };
  if (has_keys) load(k0);
  // the norm and RoPE below wait only for the small loads above
  __builtin_amdgcn_sched_barrier(0);

  auto rope = [&](float (&x)[DPL], const float4 (&g4)[DPL / 4]) {
    if (a.qk_norm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) ss += x[e] * x[e];
      ss = group_sum<LPK>(ss);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int e = 0; e < DPL; e += 4) {
        const float4 gg = g4[e / 4];
        x[e] = x[e] * inv * gg.x;
        x[e + 1] = x[e + 1] * inv * gg.y;
        x[e + 2] = x[e + 2] * inv * gg.z;
        x[e + 3] = x[e + 3] * inv * gg.w;
      }
    }
    const bool lo = dl < half;
#pragma unroll
    for (int e = 0; e < DPL / 4; ++e) {
      const float c[4] = {cs[e].x, cs[e].y, cs[e].z, cs[e].w};
      const float si[4] = {sn[e].x, sn[e].y, sn[e].z, sn[e].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float other = __shfl_xor(x[4 * e + t], LPK / 2, 64);   // channel -/+ D/2
        x[4 * e + t] = lo ? x[4 * e + t] * c[t] - other * si[t] : x[4 * e + t] * c[t] + other * si[t];
      }
    }
  };

#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (a.fused) rope(qv[j], gq);
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[j][e] *= a.scale;
  }

  // the new row of a fused step, built in registers by the last split's wave
  uint4 knew[NV], vnew[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) knew[v] = vnew[v] = make_uint4(0, 0, 0, 0);
  if (owns_new) {
    rope(kf, gk);
    KT* Kw = const_cast<KT*>(Kh) + (size_t)pos * D;
    KT* Vw = const_cast<KT*>(Vh) + (size_t)pos * D;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float t[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) t[e] = kf[v * VEC + e];
      knew[v] = pack_kv<KT, VEC>(t);
#pragma unroll
      for (int e = 0; e < VEC; ++e) t[e] = vf[v * VEC + e];
      vnew[v] = pack_kv<KT, VEC>(t);
      if (sub == 0) {
        *reinterpret_cast<uint4*>(Kw + v * VEC) = knew[v];
        *reinterpret_cast<uint4*>(Vw + v * VEC) = vnew[v];
      }
    }
  }

  float mx[R], ls[R], acc[R][DPL];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    mx[j] = -1e30f;
    ls[j] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[j][e] = 0.f;
  }
  // the new row (as stored, rounded to the cache dtype) opens the state of
  // the owner's first lane group: score s, weight 1, value v
  if (owns_new) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float d = 0.f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float kv[VEC];
        Vec16<KT>::unpack(knew[v], kv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qv[j][v * VEC + e], kv[e], d);
      }
      d = group_sum<LPK>(d);
      if (sub == 0) {
        mx[j] = d;
        ls[j] = 1.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float vv[VEC];
          Vec16<KT>::unpack(vnew[v], vv);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][v * VEC + e] = vv[e];
        }
      }
    }
  }

  for (int kb = k0; kb < kend; kb += TILE) {
    // the tile's raw rows (unpacked to float where used, to keep registers low)
    uint4 kc[U][NV], vc[U][NV];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = kb + u * KPW + sub < kend;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        kc[u][v] = kr[u][v];
        vc[u][v] = vr[u][v];
      }
    }
    if (kb + TILE < kend) load(kb + TILE);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float sc[U];
      float tmax = mx[j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float d = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float kv[VEC];
          Vec16<KT>::unpack(kc[u][v], kv);
#pragma unroll
          for (int e = 0; e < VEC; ++e) d = fmaf(qv[j][v * VEC + e], kv[e], d);
        }
        sc[u] = group_sum<LPK>(d);
        if (ok[u]) tmax = fmaxf(tmax, sc[u]);
      }
      // one rescale per tile
      const float c = expf(mx[j] - tmax);
      ls[j] *= c;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[j][e] *= c;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = ok[u] ? expf(sc[u] - tmax) : 0.f;
        ls[j] += p;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float vv[VEC];
          Vec16<KT>::unpack(vc[u][v], vv);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][v * VEC + e] = fmaf(p, vv[e], acc[j][v * VEC + e]);
        }
      }
      mx[j] = tmax;
    }
  }

  // merge the KPW key groups of the wave (lanes with equal dl): xor LPK,
  // 2 LPK, ... 32 (xor 8 within a row of 16 lanes by DPP)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      auto xch = [&](float v) { return off == 8 ? dpp<kDppRor8>(v) : __shfl_xor(v, off, 64); };
      const float om = xch(mx[j]);
      const float ol = xch(ls[j]);
      const float nm = fmaxf(mx[j], om);
      const float ca = expf(mx[j] - nm), cb = expf(om - nm);
      ls[j] = ls[j] * ca + ol * cb;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float oa = xch(acc[j][e]);
        acc[j][e] = acc[j][e] * ca + oa * cb;
      }
      mx[j] = nm;
    }
  }
  if (a.nsplit_max == 1) {
    // a single split per row and head: its state is the result (acc / l)
    if (lane < LPK) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const size_t off = ((size_t)m * a.Hq + g * R + j) * D + dl;
#pragma unroll
        for (int e = 0; e < DPL; e += 4)
          store_o4<D>(a, off + e, make_float4(acc[j][e] / ls[j], acc[j][e + 1] / ls[j],
                                            acc[j][e + 2] / ls[j], acc[j][e + 3] / ls[j]));
      }
    }
    return;
  }

  // the block's four waves merged in LDS, in wave order
  constexpr int NC = D / 4;           // float4 channel groups of a head
  constexpr int ITEMS = R * NC;       // (head, channel group) items of the block
  static_assert(ITEMS <= 256, "one item per thread at most");
  __shared__ float s_m[4][R], s_l[4][R];
  __shared__ float4 s_a[4][R][NC];
  if (lane < LPK) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int e = 0; e < DPL; e += 4)
        s_a[wave][j][(dl + e) / 4] = make_float4(acc[j][e], acc[j][e + 1], acc[j][e + 2], acc[j][e + 3]);
      if (lane == 0) {
        s_m[wave][j] = mx[j];
        s_l[wave][j] = ls[j];
      }
    }
  }
  __syncthreads();
  const int ns = (len + chunk - 1) / chunk;   // splits of this row
  const int nblk = (ns + 3) / 4;              // blocks of this (row, KV head)
  const int blk = blockIdx.x;
  const int item = tid % ITEMS, j = item / NC, c = item % NC;
  const size_t head = (size_t)m * a.Hq + g * R + j;
  if (tid < ITEMS) {
    float M = s_m[0][j];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][j]);
    float L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float cw = expf(s_m[w][j] - M);
      L = fmaf(s_l[w][j], cw, L);
      const float4 v = s_a[w][j][c];
      A = make_float4(fmaf(v.x, cw, A.x), fmaf(v.y, cw, A.y), fmaf(v.z, cw, A.z), fmaf(v.w, cw, A.w));
    }
    if (nblk == 1) {
      store_o4<D>(a, head * D + 4 * c, make_float4(A.x / L, A.y / L, A.z / L, A.w / L));
    } else {
      // the block's partial, written through to the device-coherent level so
      // that the block that merges them (on any XCD) reads the values stored
      // (deferred: plain stores, the launch boundary makes them visible)
      const size_t pb = head * a.nsplit_max + blk;
      if constexpr (DEFER) {
        *reinterpret_cast<float4*>(a.pacc + pb * D + 4 * c) = A;
        if (c == 0) *reinterpret_cast<float2*>(a.pml + pb * 2) = make_float2(M, L);
      } else {
        store_coherent4(a.pacc + pb * D + 4 * c, A);
        if (c == 0) store_coherent2(a.pml + pb * 2, M, L);
      }
    }
  }
  if (nblk == 1) return;
  if constexpr (DEFER) return;
  // ticket of this (row, KV head): the block that arrives last merges every
  // block's partial, in block order (the result does not depend on which
  // block arrives last)
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores are complete
  __shared__ int s_last;
  __syncthreads();
  if (tid == 0) {
    int* t = a.ticket + (size_t)m * a.Hkv + g;
    const int old = __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == nblk - 1;
    if (last) __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  attn_merge_states<D, R, true>(a, m, g, nblk);
}

// The deferred merge: one workgroup per (KV head, row) of a DEFER launch.
template <int D, int R>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int g = blockIdx.x, m = blockIdx.y;
  int slot, pos;
  row_of(a.rows, a.st, m, slot, pos);
  const int len = pos + 1;
  const int chunk = attn_chunk(len, a.M, a.Hkv, a.waves);
  const int nblk = ((len + chunk - 1) / chunk + 3) / 4;
  if (nblk == 1) return;   // that row's block wrote the output itself
  attn_merge_states<D, R, false>(a, m, g, nblk);
}

// ------------------------------------------------------------------ slot bookkeeping
__global__ void k_advance(SlotTables st, RowMap rows, int M) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (rows.mode == kRowsPrefill) {
    if (m == 0) st.pos[rows.slot0] = M;
  } else if (m < M) {
    st.pos[step_slot(rows, rows.row0 + m)] += 1;
  }
}

__global__ void k_slot_list(int32_t* dst, SlotListArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) dst[a.off + i] = a.v[i];
}

struct SlotSetArgs {
  void* k[kMaxLayers];
  void* v[kMaxLayers];
  int slot, cap, pos, set_ptrs;
};

__global__ void k_set_slot(SlotTables st, SlotSetArgs a) {
  const int l = threadIdx.x;
  if (a.set_ptrs && l < st.L) {
    st.kv[((size_t)a.slot * st.L + l) * 2] = a.k[l];
    st.kv[((size_t)a.slot * st.L + l) * 2 + 1] = a.v[l];
  }
  if (l == 0) {
    if (a.cap >= 0) st.cap[a.slot] = a.cap;
    if (a.pos >= 0) st.pos[a.slot] = a.pos;
  }
}

// valid rows [0, rows) of every head of every buffer, old stride -> new stride
__global__ __launch_bounds__(256) void k_kv_copy(KvCopyArgs a) {
  const int b = blockIdx.z, hk = blockIdx.y;
  const size_t row_bytes = (size_t)a.D * a.elem_bytes;
  const uint4* src = reinterpret_cast<const uint4*>(
      reinterpret_cast<const char*>(a.src[b]) + (size_t)hk * a.s_old * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.dst[b]) +
                                        (size_t)hk * a.s_new * row_bytes);
  const size_t n = (size_t)a.rows * row_bytes / 16;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = src[i];
}

// ------------------------------------------------------------------ token choice controls
__device__ __forceinline__ int ctl_step(const ChoiceCtl& c) {
  return c.step0 + (c.step_base ? *c.step_base : 0) + (c.step_ctr ? *c.step_ctr : 0);
}
// true when token i of the row may not be chosen
__device__ __forceinline__ bool ctl_masked(const ChoiceCtl& c, const uint32_t* sup_row, int i,
                                           bool eos_blocked) {
  return (sup_row && ((sup_row[i >> 5] >> (i & 31)) & 1u)) || (eos_blocked && i == c.eos);
}
// The row's final token: eos once stopped (stopped = true: the seen set is
// left alone), and the stop recorded when the choice is eos.
__device__ __forceinline__ int ctl_finish(const ChoiceCtl& c, int b, int tok, int step,
                                          bool& stopped) {
  stopped = false;
  if (c.eos_step) {
    if (c.eos_step[b] >= 0) {
      stopped = true;
      return c.eos;
    }
    if (tok == c.eos) c.eos_step[b] = step;
  }
  return tok;
}

// ------------------------------------------------------------------ argmax
struct Top2 {
  float v1, v2;
  int i1;
};

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1)) {
    r.v1 = b.v1;
    r.i1 = b.i1;
    r.v2 = fmaxf(b.v2, a.v1);
  } else {
    r.v1 = a.v1;
    r.i1 = a.i1;
    r.v2 = fmaxf(a.v2, b.v1);
  }
  return r;
}

__device__ __forceinline__ Top2 wave_top2(Top2 t) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Top2 o;
    o.v1 = __shfl_xor(t.v1, off, 64);
    o.v2 = __shfl_xor(t.v2, off, 64);
    o.i1 = __shfl_xor(t.i1, off, 64);
    t = top2_merge(t, o);
  }
  return t;
}

__global__ __launch_bounds__(256) void k_argmax_part(ArgmaxArgs a) {
  __shared__ Top2 st[4];
  const int blk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lo = blk * kArgmaxChunk, hi = min(a.V, lo + kArgmaxChunk);
  const float* z = a.z + (size_t)b * a.V;
  const uint32_t* seen = a.seen ? a.seen + (size_t)b * a.nwords : nullptr;
  const uint32_t* sup = a.ctl.suppress ? a.ctl.suppress + (size_t)b * a.nwords : nullptr;
  const int step = ctl_step(a.ctl);
  const bool eos_blocked = a.ctl.eos >= 0 && step < a.ctl.min_new;
  Top2 t{-INFINITY, -INFINITY, 0x7fffffff};
  for (int i = lo + tid; i < hi; i += 256) {
    float v = z[i];
    if (ctl_masked(a.ctl, sup, i, eos_blocked)) v = -INFINITY;
    if (seen && ((seen[i >> 5] >> (i & 31)) & 1u)) v = v > 0.f ? v / a.penalty : v * a.penalty;
    if (v > t.v1) {
      t.v2 = t.v1;
      t.v1 = v;
      t.i1 = i;
    } else if (v > t.v2) {
      t.v2 = v;
    }
  }
  t = wave_top2(t);
  if ((tid & 63) == 0) st[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) {
    Top2 r = st[0];
    for (int w = 1; w < 4; ++w) r = top2_merge(r, st[w]);
    if (a.nblk == 1) {   // one block: this is the final result (k_argmax_final is skipped)
      bool stopped;
      const int tok = ctl_finish(a.ctl, b, min(r.i1, a.V - 1), step, stopped);
      a.tok[b] = tok;
      if (a.margin) a.margin[b] = r.v1 - r.v2;
      if (a.seen && !stopped) a.seen[(size_t)b * a.nwords + (tok >> 5)] |= 1u << (tok & 31);
      return;
    }
    float* p = a.part + ((size_t)b * a.nblk + blk) * 3;
    p[0] = r.v1;
    p[1] = __int_as_float(r.i1);
    p[2] = r.v2;
  }
}

__global__ __launch_bounds__(64) void k_argmax_final(ArgmaxArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  Top2 t{-INFINITY, -INFINITY, 0x7fffffff};
  for (int k = lane; k < a.nblk; k += 64) {
    const float* p = a.part + ((size_t)b * a.nblk + k) * 3;
    t = top2_merge(t, Top2{p[0], p[2], __float_as_int(p[1])});
  }
  t = wave_top2(t);
  if (lane == 0) {
    bool stopped;
    const int tok = ctl_finish(a.ctl, b, min(t.i1, a.V - 1), ctl_step(a.ctl), stopped);
    a.tok[b] = tok;
    if (a.margin) a.margin[b] = t.v1 - t.v2;
    if (a.seen && !stopped) a.seen[(size_t)b * a.nwords + (tok >> 5)] |= 1u << (tok & 31);
  }
}


// ------------------------------------------------------------------ top-k sampling
// Unsigned order of the keys is the order of the values; -0 and +0 share a
// key.  Key 0 (a NaN pattern) marks an empty element.
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v == 0.f) v = 0.f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The selected set: keys >= t (tie false), or keys > t plus the r keys equal
// to t that come first in index order (tie true).
struct TopkSel {
  uint32_t t;
  int r;
  bool tie;
};

// Radix select of the kk-th largest key of the block (1 <= kk <= number of
// non-empty keys), four bits per pass from the top.  The count of each digit
// in a wave comes from ballots; lane b < 16 of every wave then sums bin b over
// the waves from LDS (hist: two buffers of [16 waves][16 bins], alternating,
// so one barrier per pass suffices) and every wave finds the digit itself.
// Stops early once the chosen group holds exactly the keys still wanted.
__device__ TopkSel block_select(const uint32_t (&key)[kSamplePerThread], int kk,
                                uint32_t* hist) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t P = 0;
  int r = kk;
  for (int pass = 0; pass < 8; ++pass) {
    const int s = 28 - 4 * pass;
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kSamplePerThread; ++j) {
      const bool act = key[j] != 0u && (pass == 0 || (key[j] >> (s + 4)) == P);
      if (__ballot(act) == 0) continue;
      const uint32_t d = (key[j] >> s) & 15u;
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint32_t c = (uint32_t)__popcll(__ballot(act && d == (uint32_t)b));
        if (lane == b) mine += c;
      }
    }
    uint32_t* h = hist + (pass & 1) * 256;
    if (lane < 16) h[w * 16 + lane] = mine;
    __syncthreads();
    uint32_t tot = 0;
    if (lane < 16)
      for (int v = 0; v < nw; ++v) tot += h[v * 16 + lane];
    uint32_t incl = tot;   // lane b < 16: keys of the group in bins >= b
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t o = __shfl_down(incl, off, 64);
      if (lane + off < 16) incl += o;
    }
    const uint32_t above = incl - tot;
    const uint64_t hit = __ballot(lane < 16 && above < (uint32_t)r && (uint32_t)r <= incl);
    const int d = hit ? __builtin_ctzll(hit) : 0;
    const uint32_t td = __shfl(tot, d, 64);
    r -= (int)__shfl(above, d, 64);
    P = (P << 4) | (uint32_t)d;
    if (td == (uint32_t)r) return TopkSel{P << s, r, false};
  }
  return TopkSel{P, r, true};
}

// Exclusive prefix sum over the block in thread order of small values whose
// set bits all lie in MASK, and the block's total: one ballot per bit gives
// the wave's prefix (mbcnt) and total; sbuf holds one word per wave.
template <uint32_t MASK>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sbuf,
                                                    uint32_t* total = nullptr) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t pre = 0, wtot = 0;
#pragma unroll
  for (int bit = 0; bit < 32; ++bit) {
    if (!((MASK >> bit) & 1u)) continue;
    const uint64_t m = __ballot((v >> bit) & 1u);
    pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))
           << bit;
    wtot += (uint32_t)__popcll(m) << bit;
  }
  if (lane == 0) sbuf[w] = wtot;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int v2 = 0; v2 < nw; ++v2) {
    const uint32_t x = sbuf[v2];
    base += v2 < w ? x : 0u;
    tot += x;
  }
  if (total) *total = tot;
  return base + pre;
}

// Writes the selected (key, index) pairs to dst[0..kk) in index order
// (thread t holds elements t*e .. t*e+e-1).
__device__ void compact_selected(const uint32_t (&key)[kSamplePerThread],
                                 const uint32_t (&idx)[kSamplePerThread], TopkSel sel, int kk,
                                 uint2* dst, uint32_t* sbuf) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) {
    if (key[j] == 0u) continue;
    if (sel.tie ? key[j] > sel.t : key[j] >= sel.t) ++gt;
    else if (sel.tie && key[j] == sel.t) ++eq;
  }
  const uint32_t base = block_excl_scan<0x000F000Fu>(gt | (eq << 16), sbuf);
  uint32_t gb = base & 0xffffu, eb = base >> 16;
  const uint32_t r = (uint32_t)sel.r;
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) {
    if (key[j] == 0u) continue;
    if (sel.tie ? key[j] > sel.t : key[j] >= sel.t) {
      const uint32_t slot = gb + min(eb, r);
      ++gb;
      if (slot < (uint32_t)kk) dst[slot] = make_uint2(key[j], idx[j]);
    } else if (sel.tie && key[j] == sel.t) {
      if (eb < r && gb + eb < (uint32_t)kk) dst[gb + eb] = make_uint2(key[j], idx[j]);
      ++eb;
    }
  }
}

// Keys of this thread's elements of row b, chunk [lo, lo + n): penalised
// logits, indices implicit.
__device__ __forceinline__ void load_logit_keys(const SampleArgs& a, int b, int lo, int n,
                                                uint32_t (&key)[kSamplePerThread],
                                                uint32_t (&idx)[kSamplePerThread]) {
  const int e = (n + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * e;
  const float* z = a.z + (size_t)b * a.V + lo;
  const uint32_t* seen = a.seen ? a.seen + (size_t)b * a.nwords : nullptr;
  const uint32_t* sup = a.ctl.suppress ? a.ctl.suppress + (size_t)b * a.nwords : nullptr;
  const bool eos_blocked = a.ctl.eos >= 0 && ctl_step(a.ctl) < a.ctl.min_new;
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) {
    key[j] = 0u;
    idx[j] = 0u;
    const int i = i0 + j;
    if (j < e && i < n) {
      float v = z[i];
      const int g = lo + i;
      if (ctl_masked(a.ctl, sup, g, eos_blocked)) v = -INFINITY;
      if (seen && ((seen[g >> 5] >> (g & 31)) & 1u)) v = v > 0.f ? v / a.penalty : v * a.penalty;
      key[j] = order_key(v);
      idx[j] = (uint32_t)g;
    }
  }
}

// Chunk blk of row b -> its top-k candidates in part (index order; slots past
// the chunk's length hold empty keys).
__global__ __launch_bounds__(kSampleThreads) void k_sample_part(SampleArgs a) {
  __shared__ uint32_t hist[512];
  __shared__ uint32_t sbuf[kSampleThreads / 64];
  const int blk = blockIdx.x, b = blockIdx.y;
  const int lo = blk * kSampleChunk, n = min(a.V - lo, kSampleChunk);
  uint32_t key[kSamplePerThread], idx[kSamplePerThread];
  load_logit_keys(a, b, lo, n, key, idx);
  const int kk = min(a.k, n);
  const TopkSel sel = block_select(key, kk, hist);
  uint2* dst = a.part + ((size_t)b * a.nblk + blk) * a.k;
  compact_selected(key, idx, sel, kk, dst, sbuf);
  const int t = threadIdx.x;
  if (t >= kk && t < a.k) dst[t] = make_uint2(0u, 0u);
}

// Rank of (value `mine`, position p) in list[0..n): the number of entries
// with a larger value, or an equal value at an earlier position -- one
// unsigned compare of (value << 32 | ~position) pairs.  Called by whole waves
// (lanes past the list pass anything); each wave walks the list 64 values at
// a time, broadcasting one value per step from a register (an immediate lane
// index).  Entries past the list read as value 0 at positions after p, which
// never count.
template <typename Get>
__device__ __forceinline__ int list_rank(Get get, int n, uint32_t mine, int p) {
  const int lane = threadIdx.x & 63;
  const uint64_t me = ((uint64_t)mine << 32) | (uint32_t)~p;
  int rank = 0;
  for (int base = 0; base < n; base += 64) {
    const uint32_t kl = base + lane < n ? get(base + lane) : 0u;
#pragma unroll
    for (int jj = 0; jj < 64; ++jj) {
      const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)kl, jj) << 32) |
                          (uint32_t)~(base + jj);
      rank += kj > me ? 1 : 0;
    }
  }
  return rank;
}

// Candidates cand[0..n) (index order) -> sorted[rank] for the ranks below kk.
__device__ __forceinline__ void rank_candidates(const uint2* cand, int n, int kk, uint2* sorted) {
  const int t = threadIdx.x, lane = t & 63;
  if (t - lane >= n) return;   // the whole wave is past the list
  const uint2 me = t < n ? cand[t] : make_uint2(0u, 0u);
  const int rank = list_rank([&](int j) { return cand[j].x; }, n, me.x, t);
  if (t < n && rank < kk) sorted[rank] = me;
}

// Prefiltered candidates ranked directly (above this the radix select runs)
constexpr int kSampleCandMax = 512;

// Row b: the top-k set (from the logits, or from the chunks' candidates),
// sorted by key descending and index ascending, then the draw: weights
// exp((v - v_max) / temperature) summed in that order, the shortest prefix
// whose weight reaches top_p of the total, and the first candidate whose
// running sum exceeds u times the prefix's weight.
//
// The set: groups of g consecutive threads (g the largest power of two <= 64
// leaving at least 2k groups) each hold a maximum; the k-th largest of these
// maxima (k distinct keys) is at most the k-th largest key, so the keys at
// or above it contain the set.  When they are few they are ranked directly;
// otherwise (ties, or k close to the number of groups) the radix select
// finds the set.
__global__ __launch_bounds__(kSampleThreads) void k_sample_final(SampleArgs a) {
  __shared__ uint32_t hist[512];
  __shared__ uint32_t sbuf[kSampleThreads / 64];
  __shared__ uint32_t gmax[kSampleThreads / 2];
  __shared__ uint32_t bound;
  __shared__ uint2 cand[kSampleCandMax];
  __shared__ uint2 sorted[kTopKMax];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63;
  uint32_t key[kSamplePerThread], idx[kSamplePerThread];
  if (a.nblk == 1) {
    load_logit_keys(a, b, 0, a.V, key, idx);
  } else {
    const int n = a.nblk * a.k;
    const int e = (n + blockDim.x - 1) / blockDim.x;
    const uint2* src = a.part + (size_t)b * n;
#pragma unroll
    for (int j = 0; j < kSamplePerThread; ++j) {
      const int i = t * e + j;
      uint2 c = make_uint2(0u, 0u);
      if (j < e && i < n) c = src[i];
      key[j] = c.x;
      idx[j] = c.y;
    }
  }
  const int kk = a.k;

  // lower bound of the k-th largest key: the k-th largest group maximum
  int g = 64;
  while (g > 2 && (int)blockDim.x / g < 2 * kk) g >>= 1;
  const int G = blockDim.x / g;
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) m = max(m, key[j]);
  for (int off = 1; off < g; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((lane & (g - 1)) == 0) gmax[t / g] = m;
  __syncthreads();
  if (t - lane < G) {
    const uint32_t v = t < G ? gmax[t] : 0u;
    const int r = list_rank([&](int j) { return gmax[j]; }, G, v, t);
    if (t < G && r == kk - 1) bound = v;
  }
  __syncthreads();
  const uint32_t L = bound;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) mine += (key[j] != 0u && key[j] >= L) ? 1u : 0u;
  uint32_t nc = 0;
  const uint32_t base = block_excl_scan<0xFu>(mine, sbuf, &nc);
  if (nc <= (uint32_t)kSampleCandMax) {
    uint32_t slot = base;
#pragma unroll
    for (int j = 0; j < kSamplePerThread; ++j)
      if (key[j] != 0u && key[j] >= L) cand[slot++] = make_uint2(key[j], idx[j]);
    __syncthreads();
    rank_candidates(cand, (int)nc, kk, sorted);
  } else {
    if (t < kTopKMax) cand[t] = make_uint2(0u, 0u);
    const TopkSel sel = block_select(key, kk, hist);   // its barriers order the clear above
    compact_selected(key, idx, sel, kk, cand, sbuf);
    __syncthreads();
    rank_candidates(cand, kk, kk, sorted);
  }
  __syncthreads();
  if (t >= 64) return;
  const float vmax = key_value(sorted[0].x);
  float c[4];
  float run = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane * 4 + q;
    float p = 0.f;
    if (i < kk && sorted[i].x != 0u) p = expf((key_value(sorted[i].x) - vmax) / a.temperature);
    run += p;
    c[q] = run;
  }
  const float incl = wave_incl_scan(run);
  const float excl = incl - run;
#pragma unroll
  for (int q = 0; q < 4; ++q) c[q] += excl;
  const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
  int mcut = kk;
  float mass = total;
  if (a.top_p < 1.f) {
    const float thr = a.top_p * total;
    int qf = 4;
    float cf = 0.f;
#pragma unroll
    for (int q = 3; q >= 0; --q)
      if (lane * 4 + q < kk && c[q] >= thr) {
        qf = q;
        cf = c[q];
      }
    const uint64_t hb = __ballot(qf < 4);
    if (hb) {
      const int Lq = __builtin_ctzll(hb);
      mcut = Lq * 4 + __builtin_amdgcn_readlane(qf, Lq) + 1;
      mass = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cf), Lq));
    }
  }
  const float u = a.u[(size_t)(a.u_row ? *a.u_row : 0) * a.u_stride + b];
  const float target = u * mass;
  int qd = 4;
#pragma unroll
  for (int q = 3; q >= 0; --q)
    if (lane * 4 + q < mcut && c[q] > target) qd = q;
  const uint64_t hd = __ballot(qd < 4);
  int pos = mcut - 1;
  if (hd) {
    const int Lq = __builtin_ctzll(hd);
    pos = Lq * 4 + __builtin_amdgcn_readlane(qd, Lq);
  }
  if (lane == 0) {
    bool stopped;
    const int tok = ctl_finish(a.ctl, b, min((int)sorted[pos].y, a.V - 1), ctl_step(a.ctl), stopped);
    a.tok[b] = tok;
    if (a.seen && !stopped) a.seen[(size_t)b * a.nwords + (tok >> 5)] |= 1u << (tok & 31);
  }
}

// ------------------------------------------------------------------ MFMA path
typedef __bf16 Bf16x8 __attribute__((ext_vector_type(8)));
typedef float Floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Bf16x8 as_bf16x8(uint4 v) {
  union {
    uint4 u;
    Bf16x8 b;
  } c;
  c.u = v;
  return c.b;
}

// Split-K GEMM of the rows of a call, in row tiles of 64: part[split, m, n] =
// sum over the split's K range of (hi + lo)[m, k] * W[n, k]: bf16 MFMA
// 16x16x32, float32 accumulation.  Workgroup (64 weight rows, split, row
// tile): wave w owns 16 weight rows.  The
// split is walked in 64-wide stages; each stage's activation tile (64 rows,
// hi and lo) is read with row-contiguous loads into a double-buffered LDS
// tile, from which every wave reads its MFMA fragments, while the weight
// fragments go straight to registers.  Both come through a P-deep register
// ring, so the loads of P stages are in flight while a stage is multiplied,
// and the in-order memory counter only ever waits for the oldest stage.
// NCH > 0: every workgroup walks exactly NCH stages, fully unrolled, with
// every load issued unconditionally (clamped addresses; groups past the split
// end are zeroed when written to LDS), so the compiler's counter waits are
// exact (with the stage loop it waited for every outstanding load at the
// loop head: measured 12-32% slower on the 64-row shapes).  NCH = 0: the
// stage loop, for other stage counts.
template <int P, int NCH>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  // LDS tile [buf][hi/lo][row][8 x 16 bytes]; the 16-byte chunk c of row r
  // sits at c ^ (r & 7) so that a fragment read spreads over the banks
  __shared__ uint4 sa[2][2][kMmaRows][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kMmaBlockN + wave * 16, split = blockIdx.y;
  const int r0 = blockIdx.z * kMmaRows;   // the workgroup's row tile
  const int K = a.K;
  const int kb = split * a.kc, ke = min(K, kb + a.kc);
  const int nch = (ke - kb + kMmaCh - 1) / kMmaCh;

  const int row = n0 + li;
  const int sg = row < a.seg_end[0] ? 0 : (row < a.seg_end[1] ? 1 : 2);
  const int sb = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
  // rows past N read row 0 of the segment (in bounds); their sums are not stored
  const uint16_t* wp = reinterpret_cast<const uint16_t*>(pick3(a.W, sg)) +
                       (size_t)(row < a.N ? row - sb : 0) * K + lg * 8;
  // staging: thread -> rows srow and srow + 32, 16-byte group sc
  const int srow = tid >> 3, sc = tid & 7;
  const uint16_t* sh = a.hi + (size_t)(r0 + srow) * K + sc * 8;
  const uint16_t* sl = a.lo + (size_t)(r0 + srow) * K + sc * 8;

  uint4 ar[P][4], wr[P][2];
  auto issue_a = [&](int p, int c) {
    const int k = kb + c * kMmaCh + sc * 8;
    const bool ok = k < ke;   // whole groups: K and the split ends are multiples of 32
    const int kk = ok ? k - sc * 8 : 0;
    const uint4 z = make_uint4(0, 0, 0, 0);
    ar[p][0] = ok ? ldg16(sh + kk) : z;
    ar[p][1] = ok ? ldg16(sh + (size_t)32 * K + kk) : z;
    ar[p][2] = ok ? ldg16(sl + kk) : z;
    ar[p][3] = ok ? ldg16(sl + (size_t)32 * K + kk) : z;
  };
  auto issue_w = [&](int p, int c) {
    // stages past the split end read in-bounds weights that meet zero activations
#pragma unroll
    for (int s = 0; s < 2; ++s) wr[p][s] = ldg16(wp + min(kb + c * kMmaCh + s * 32, K - 32));
  };
  Floatx4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = Floatx4{0.f, 0.f, 0.f, 0.f};
  // one stage's MFMAs on LDS buffer buf with the weights of ring slot p
  auto mma_stage = [&](int p, int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int pos = (s * 4 + lg) ^ (li & 7);
      const Bf16x8 b = as_bf16x8(wr[p][s]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sa[buf][0][i * 16 + li][pos]), b,
                                                         acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sa[buf][1][i * 16 + li][pos]), b,
                                                         acc[i], 0, 0, 0);
      }
    }
  };
  if constexpr (NCH > 0) {
    auto issue_a_all = [&](int p, int c) {
      const int kk = min(kb + c * kMmaCh + sc * 8, K - 8) - sc * 8;
      ar[p][0] = ldg16(sh + kk);
      ar[p][1] = ldg16(sh + (size_t)32 * K + kk);
      ar[p][2] = ldg16(sl + kk);
      ar[p][3] = ldg16(sl + (size_t)32 * K + kk);
    };
#pragma unroll
    for (int p = 0; p < P && p < NCH; ++p) {
      issue_a_all(p, p);
      issue_w(p, p);
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int p = c % P, buf = c & 1;
      const int sw = sc ^ (srow & 7);
      // whole groups: K and the split ends are multiples of 32 (a mask, not a
      // select: a select of the register ring became a scratch access)
      const uint32_t mk = 0u - (uint32_t)(kb + c * kMmaCh + sc * 8 < ke);
      auto keep = [mk](uint4 v) { return make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk); };
      sa[buf][0][srow][sw] = keep(ar[p][0]);
      sa[buf][0][srow + 32][sw] = keep(ar[p][1]);
      sa[buf][1][srow][sw] = keep(ar[p][2]);
      sa[buf][1][srow + 32][sw] = keep(ar[p][3]);
      __syncthreads();
      if (c + P < NCH) issue_a_all(p, c + P);
      mma_stage(p, buf);
      if (c + P < NCH) issue_w(p, c + P);
    }
  } else {
#pragma unroll
  for (int p = 0; p < P; ++p) {
    issue_a(p, p);
    issue_w(p, p);
  }
  for (int c0 = 0; c0 < nch; c0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + p;
      if (c < nch) {
        const int buf = c & 1;
        const int sw = sc ^ (srow & 7);
        sa[buf][0][srow][sw] = ar[p][0];
        sa[buf][0][srow + 32][sw] = ar[p][1];
        sa[buf][1][srow][sw] = ar[p][2];
        sa[buf][1][srow + 32][sw] = ar[p][3];
        __syncthreads();
        issue_a(p, c + P);
        mma_stage(p, buf);
        issue_w(p, c + P);
      }
    }
  }
  }
  // C layout: column li, rows 4 * lg + r of each 16x16 tile
  if (row < a.N) {
    float* Pp = a.part + ((size_t)split * a.mrows + r0) * a.N + row;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) Pp[(size_t)(i * 16 + lg * 4 + r) * a.N] = acc[i][r];
  }
}

// Split-K GEMM of a prefill chunk over 128 x 128 output tiles: part[split,
// m, n] = sum over the split's K range of (hi + lo)[m, k] * W[n, k] (bf16 MFMA
// 16x16x32, float32 accumulation), as k_gemm, for calls of more than one
// 64-row tile.  Workgroup (128 rows x 128 weight rows, split): wave (wm, wn)
// owns rows wm*64.. and weight rows wn*64.. (4 x 4 MFMA tiles).  Both operand
// tiles (activation hi and lo, weights) pass through a double-buffered LDS
// tile in 32-wide stages, the loads of the next stages (up to four) in a
// register ring during the math; a stage costs a wave 12 fragment reads for
// 32 MFMAs, where the
// 64 x 64 tile of k_gemm pays one per MFMA and re-reads each activation tile
// for every 64 weight rows.  The linear workgroup id is remapped so that each
// XCD (workgroups go round-robin over the 8, each with its own L2) walks one
// contiguous range of (row tile fastest, then split, then weight tile).
template <int NST>
__global__ __launch_bounds__(256) void k_gemm_tile(GemmArgs a) {
  constexpr int BM = 128, BN = 128, BK = 32;
  // NST > 0: every workgroup walks NST stages, fully unrolled, through a
  // P-deep register ring (loads of P stages in flight; stages past the split
  // end read in-bounds data and are zeroed at the LDS write); NST = 0: a
  // stage loop with one stage in flight
  constexpr int P = NST == 0 ? 1 : (NST < 4 ? NST : 4);
  // [buf][act hi, act lo, weights][row][4 chunks of 16 bytes]; chunk c of row
  // r sits at c ^ ((r >> 1) & 3), so a fragment read (16 rows, 4 chunks)
  // spreads over the banks
  __shared__ uint4 sm[2][3][BM][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int nrt = (a.mrows + BM - 1) / BM;
  int rt, split, wt;
  {
    int b = blockIdx.x;
    const int t8 = gridDim.x & ~7;
    if (b < t8) b = (b & 7) * (t8 >> 3) + (b >> 3);
    rt = b % nrt;
    b /= nrt;
    split = b % a.ks;
    wt = b / a.ks;
  }
  const int K = a.K;
  const int kb = split * a.kc, ke = min(K, kb + a.kc);
  const int nst = NST > 0 ? NST : (ke - kb) / BK;   // K and split ends: multiples of 32

  // staging: thread -> rows sr and sr + 64 of each operand tile, chunk sc;
  // rows past the call's rows (or past N) read an in-bounds row whose
  // results are not stored
  const int sr = tid >> 2, sc = tid & 3;
  const int sw = sc ^ ((sr >> 1) & 3);
  const int m0 = min(rt * BM + sr, a.mrows - 1), m1 = min(rt * BM + sr + 64, a.mrows - 1);
  const uint16_t* h0 = a.hi + (size_t)m0 * K + sc * 8;
  const uint16_t* h1 = a.hi + (size_t)m1 * K + sc * 8;
  const uint16_t* l0 = a.lo + (size_t)m0 * K + sc * 8;
  const uint16_t* l1 = a.lo + (size_t)m1 * K + sc * 8;
  auto wrow = [&](int n) {
    const int sg = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
    const int sb = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
    return reinterpret_cast<const uint16_t*>(pick3(a.W, sg)) + (size_t)(n < a.N ? n - sb : 0) * K +
           sc * 8;
  };
  const uint16_t* w0 = wrow(wt * BN + sr);
  const uint16_t* w1 = wrow(wt * BN + sr + 64);

  uint4 ra[P][4], rb[P][2];
  auto issue = [&](int p, int c) {
    const int k = min(kb + c * BK, K - BK);
    ra[p][0] = ldg16(h0 + k);
    ra[p][1] = ldg16(h1 + k);
    ra[p][2] = ldg16(l0 + k);
    ra[p][3] = ldg16(l1 + k);
    rb[p][0] = ldg16(w0 + k);
    rb[p][1] = ldg16(w1 + k);
  };
  Floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Floatx4{0.f, 0.f, 0.f, 0.f};
  const int pos = lg ^ ((li >> 1) & 3);
  // ring slot p to LDS buffer buf; activations of stages past the split end
  // are zeroed (a mask, not a select of the ring)
  auto put = [&](int p, int buf, int c) {
    const uint32_t mk = 0u - (uint32_t)(kb + c * BK < ke);
    auto keep = [mk](uint4 v) { return make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk); };
    sm[buf][0][sr][sw] = keep(ra[p][0]);
    sm[buf][0][sr + 64][sw] = keep(ra[p][1]);
    sm[buf][1][sr][sw] = keep(ra[p][2]);
    sm[buf][1][sr + 64][sw] = keep(ra[p][3]);
    sm[buf][2][sr][sw] = rb[p][0];
    sm[buf][2][sr + 64][sw] = rb[p][1];
  };
  auto mma = [&](int buf) {
    Bf16x8 bw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bw[j] = as_bf16x8(sm[buf][2][wn * 64 + j * 16 + li][pos]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Bf16x8 ah = as_bf16x8(sm[buf][0][wm * 64 + i * 16 + li][pos]);
      const Bf16x8 al = as_bf16x8(sm[buf][1][wm * 64 + i * 16 + li][pos]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  if constexpr (NST > 0) {
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p, p);
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      const int p = c % P, buf = c & 1;
      put(p, buf, c);
      __syncthreads();
      if (c + P < NST) issue(p, c + P);
      mma(buf);
    }
  } else {
    issue(0, 0);
    for (int c = 0; c < nst; ++c) {
      const int buf = c & 1;
      put(0, buf, c);
      __syncthreads();
      issue(0, min(c + 1, nst - 1));   // the last stage re-reads itself (unused)
      mma(buf);
    }
  }
  // C layout: column li (weight row), rows 4 lg + r (activation rows)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = wt * BN + wn * 64 + j * 16 + li;
    if (n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = rt * BM + wm * 64 + i * 16 + 4 * lg + r;
        if (m < a.mrows) a.part[((size_t)split * a.mrows + m) * a.N + n] = acc[i][j][r];
      }
  }
}

// out = epi(sum over splits, in order); one thread per (row, column).
template <int EPI>
__global__ __launch_bounds__(256) void k_reduce(ReduceArgs a) {
  const int m = blockIdx.y, tid = threadIdx.x;
  const int n = blockIdx.x * 256 + tid;
  const int NO = EPI == kRedSwiglu ? a.N / 2 : a.N;
  if constexpr (EPI == kRedResidual) {
    float t = 0.f;
    if (n < NO) {
      float v = 0.f;
      for (int s = 0; s < a.ks; ++s) v += a.part[((size_t)s * a.mrows + m) * a.N + n];
      float* o = a.out + (size_t)m * a.ldo + n;
      t = *o + v;
      *o = t;
      const size_t ho = a.frag ? frag_off(m, n) : (size_t)m * a.N + n;
      split_hi_lo(t * a.gain[n], a.hi[ho], a.lo[ho]);
    }
    // one sum of squares per kSsCols = 16 columns (16 lanes)
    const float sq = group_sum<16>(t * t);
    const int b = (blockIdx.x * 256 + tid) / kSsCols;
    if ((tid & 15) == 0 && b < a.nss) a.ss[(size_t)m * a.nss + b] = sq;
    return;
  }
  // the row's norm factor: the wave's lanes add strided parts of its sums
  // of squares, then the wave's sum (the same in every lane)
  float inv = 1.f;
  if (a.ss) {
    float ss = 0.f;
    for (int b = tid & 63; b < a.nss; b += 64) ss += a.ss[(size_t)m * a.nss + b];
    ss = wave_sum(ss);
    inv = 1.0f / sqrtf(ss / (float)a.hn + a.eps);
  }
  if constexpr (EPI == kRedStore) {
    if (a.y_out)
      for (int j = n; j < a.hn; j += gridDim.x * 256)
        a.y_out[(size_t)m * a.hn + j] = a.x[(size_t)m * a.hn + j] * inv * a.gain[j];
  }
  if (n >= NO) return;
  if constexpr (EPI == kRedSwiglu) {
    float g = 0.f, u = 0.f;
    for (int s = 0; s < a.ks; ++s) {
      const float* P = a.part + ((size_t)s * a.mrows + m) * a.N;
      g += P[n];
      u += P[NO + n];
    }
    g *= inv;
    u *= inv;
    const size_t ho = a.frag ? frag_off(m, n) : (size_t)m * NO + n;
    split_hi_lo(g / (1.0f + expf(-g)) * u, a.hi[ho], a.lo[ho]);
  } else {
    float v = 0.f;
    for (int s = 0; s < a.ks; ++s) v += a.part[((size_t)s * a.mrows + m) * a.N + n];
    v *= inv;
    const int sg = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
    const int sb = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
    const float* b = pick3(a.bias, sg);
    a.out[(size_t)m * a.ldo + n] = b ? v + b[n - sb] : v;
  }
}

// The same epilogues with 4 consecutive columns per thread (16-byte partial
// and residual accesses, 8-byte hi / lo stores), for N (N / 2 for SwiGLU) a
// multiple of 4.  Each column's splits are still added in order; a wave
// covers one 256-column block and writes the sums of squares of its
// 16-column groups (residual).
template <int EPI>
__global__ __launch_bounds__(256) void k_reduce4(ReduceArgs a) {
  const int m = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int n = (blockIdx.x * 256 + tid) * 4;
  const int NO = EPI == kRedSwiglu ? a.N / 2 : a.N;
  auto sum_parts = [&](int col) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < a.ks; ++s) {
      const float4 p = *reinterpret_cast<const float4*>(a.part + ((size_t)s * a.mrows + m) * a.N + col);
      v.x += p.x;
      v.y += p.y;
      v.z += p.z;
      v.w += p.w;
    }
    return v;
  };
  // off = m * width + column, the column a multiple of 4 (fragment order:
  // the four values stay contiguous)
  auto store_hi_lo = [&](const float (&v)[4], size_t off) {
    if (a.frag) {
      const int width = EPI == kRedSwiglu ? a.N / 2 : a.N;
      off = frag_off(m, (int)(off - (size_t)m * width));
    }
    uint16_t hv[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_hi_lo(v[i], hv[i], lv[i]);
    *reinterpret_cast<uint2*>(a.hi + off) =
        make_uint2(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16));
    *reinterpret_cast<uint2*>(a.lo + off) =
        make_uint2(lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16));
  };
  if constexpr (EPI == kRedResidual) {
    float sq = 0.f;
    if (n < NO) {
      const float4 v = sum_parts(n);
      float4* o = reinterpret_cast<float4*>(a.out + (size_t)m * a.ldo + n);
      float4 t = *o;
      t.x += v.x;
      t.y += v.y;
      t.z += v.z;
      t.w += v.w;
      *o = t;
      const float4 g = *reinterpret_cast<const float4*>(a.gain + n);
      const float xg[4] = {t.x * g.x, t.y * g.y, t.z * g.z, t.w * g.w};
      store_hi_lo(xg, (size_t)m * a.N + n);
      sq = (t.x * t.x + t.y * t.y) + (t.z * t.z + t.w * t.w);
    }
    // one sum of squares per kSsCols = 16 columns (4 lanes)
    sq = group_sum<4>(sq);
    const int b = (blockIdx.x * 256 + tid) * 4 / kSsCols;
    if ((lane & 3) == 0 && b < a.nss) a.ss[(size_t)m * a.nss + b] = sq;
    return;
  }
  // the row's norm factor: the wave's lanes add strided parts of its sums
  // of squares, then the wave's sum (the same in every lane)
  float inv = 1.f;
  if (a.ss) {
    float ss = 0.f;
    for (int b = tid & 63; b < a.nss; b += 64) ss += a.ss[(size_t)m * a.nss + b];
    ss = wave_sum(ss);
    inv = 1.0f / sqrtf(ss / (float)a.hn + a.eps);
  }
  if constexpr (EPI == kRedStore) {
    if (a.y_out)
      for (int j = blockIdx.x * 256 + tid; j < a.hn; j += gridDim.x * 256)
        a.y_out[(size_t)m * a.hn + j] = a.x[(size_t)m * a.hn + j] * inv * a.gain[j];
  }
  if (n >= NO) return;
  if constexpr (EPI == kRedSwiglu) {
    const float4 g4 = sum_parts(n), u4 = sum_parts(NO + n);
    const float gs[4] = {g4.x * inv, g4.y * inv, g4.z * inv, g4.w * inv};
    const float us[4] = {u4.x * inv, u4.y * inv, u4.z * inv, u4.w * inv};
    float act[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) act[i] = gs[i] / (1.0f + expf(-gs[i])) * us[i];
    store_hi_lo(act, (size_t)m * NO + n);
  } else {
    float4 v = sum_parts(n);
    v.x *= inv;
    v.y *= inv;
    v.z *= inv;
    v.w *= inv;
    // segment ends are multiples of 4: the 4 columns share a segment
    const int sg = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
    const int sb = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
    const float* b = pick3(a.bias, sg);
    if (b) {
      const float4 bb = *reinterpret_cast<const float4*>(b + (n - sb));
      v.x += bb.x;
      v.y += bb.y;
      v.z += bb.z;
      v.w += bb.w;
    }
    *reinterpret_cast<float4*>(a.out + (size_t)m * a.ldo + n) = v;
  }
}

// ------------------------------------------------------------------ weights in B-operand order
// One thread per 16-byte chunk of the destination: chunk c is lane c % 64 of
// K step (c / 64) % (K / 32) of block c / (64 K / 32).
__global__ __launch_bounds__(256) void k_swizzle_b(SwizzleArgs a) {
  const int nks = a.K / 32;
  const size_t nblk = bfrag_blocks(a.N, a.swiglu != 0);
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nblk * nks * 64) return;
  const int lane = (int)(c % 64), li = lane & 15, lg = lane >> 4;
  const int ks = (int)((c / 64) % nks);
  const int blk = (int)(c / 64 / nks);
  const uint16_t* base;
  int row;
  bool valid;
  if (a.swiglu) {
    const int F = a.N / 2, t = blk / 4, j = blk % 4;
    row = t * 32 + (j & 1) * 16 + li;
    valid = row < F;
    base = j < 2 ? a.src[0] : a.src[1];
  } else {
    const int n = blk * 16 + li;
    valid = n < a.N;
    const int sg = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
    const int sb = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
    base = pick3(a.src, sg);
    row = n - sb;
  }
  const uint4 v = valid ? ldg16(base + (size_t)row * a.K + ks * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint4*>(a.dst + c * 8) = v;
}

// ------------------------------------------------------------------ decode GEMM, reduction inside
// GEMM of one 64-row tile (the rows of up to 64 decode streams, or a short
// prefill chunk) with its split-K reduction and epilogue in the same launch:
// C[m, n] = sum_k (hi + lo)[m, k] W[n, k], bf16 MFMA 16x16x32 with float32
// accumulation.  Workgroup (column tile of CB 16-column blocks, split) of
// eight waves: they take the split's 32-wide K steps in turn (wave w steps
// w, w + 8, ...) and each computes the whole tile over its steps.  A wave
// loads its fragments straight into registers, each a contiguous 1 KB run:
// the weights (held in B-operand order) from memory, the activations (held
// in MFMA-fragment order) mostly from L2.  Eight waves with few steps each keep every wave's chain of memory
// round trips short; there is no LDS staging and no barrier in the loop.
// The waves' tiles are added in LDS in a fixed order (w + (w + 4), then
// 0..3).  Narrow tiles give a matrix more workgroups for the same split
// count (fewer, smaller split tiles to merge) at the price of reading the
// activations once per tile.  With several splits each workgroup writes its
// tile at the device-coherent level and takes the tile's ticket; the last to
// arrive adds the ks tiles in split order (so the sum never depends on the
// arrival order) and applies the epilogue.  kDecSwiglu tiles hold CB / 2
// blocks of gate rows, then the matching up rows.
template <int NKS, int EPI, int CB>
__global__ __launch_bounds__(512) void k_gemm_dec(DecGemmArgs a) {
  constexpr int NWV = kDecWaves, NT = 64 * NWV;
  constexpr int DMAX = CB == 4 ? 3 : 4;
  constexpr int DEPTH = NKS < DMAX ? NKS : DMAX;   // K steps of loads in flight per wave
  constexpr int TC = 16 * CB;                      // tile columns
  constexpr bool SW = EPI == kDecSwiglu;
  // epilogue items: a float4 column group of a row (SwiGLU: a gate group and
  // the matching up group); TPR items a row, IT items a tile, NH per thread
  constexpr int TPR = SW ? TC / 8 : TC / 4;
  constexpr int IT = kMmaRows * TPR;
  constexpr int NH = (IT + NT - 1) / NT;
  constexpr int AT = IT < NT ? IT : NT;             // threads with items
  constexpr int NV = SW ? 2 : 1;                    // float4 values an item
  static_assert(!SW || CB % 2 == 0, "SwiGLU tiles pair gate and up blocks");
  static_assert(EPI == kDecParts || EPI == kDecResidual || NH == 1, "one item per thread");
  __shared__ float4 s_t[4][kMmaRows][TC / 4];   // four partial tiles
  __shared__ float s_inv[kMmaRows];              // the rows' norm factors
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int K = a.K;
  const int kb = split * a.kc, ke = min(K, kb + a.kc);

  // the lane's weight fragments: block tile * CB + j (blocks past the matrix
  // read its last block; their sums are never stored), K step s at s * 512
  const int nks_all = K / kDecKStep;
  const uint16_t* wblk[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j)
    wblk[j] = a.Wb + (size_t)min(tile * CB + j, a.nblk - 1) * nks_all * 512 + lane * 8;

  uint4 wv[DEPTH][CB], av[DEPTH][4][2];
  // K step t of this wave: weights first, then the activations (a 1 KB run
  // per fragment; addresses clamped into the matrix)
  auto issue = [&](int d, int t) {
    const int k = min(kb + (t * NWV + wave) * kDecKStep, K - kDecKStep);
#pragma unroll
    for (int j = 0; j < CB; ++j) wv[d][j] = ldg16_nt(wblk[j] + (size_t)(k >> 5) * 512);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t f = ((size_t)((k >> 5) * 4 + i) * 64 + lane) * 8;
      av[d][i][0] = ldg16(a.hi + f);
      av[d][i][1] = ldg16(a.lo + f);
    }
  };
  Floatx4 acc[4][CB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = Floatx4{0.f, 0.f, 0.f, 0.f};
  // the norm factor inv_m of every row (store and SwiGLU epilogues): wave w
  // takes rows 8 w .. 8 w + 7, eight lanes a row, each adding every eighth
  // of the row's sums of squares; their loads go out ahead of the operands
  constexpr bool NORMED = EPI == kDecStore || EPI == kDecSwiglu;
  constexpr int SSL = 16;   // sums a lane loads in the first pass
  const int rr = wave * 8 + (lane >> 3), rq = lane & 7;
  float ssv[SSL];
  const float* sp = NORMED && a.ss_in ? a.ss_in + (size_t)min(rr, a.M - 1) * a.nss_in : nullptr;
  if constexpr (NORMED) {
#pragma unroll
    for (int i = 0; i < SSL; ++i) {
      const int b = rq + 8 * i;
      ssv[i] = sp && b < a.nss_in ? sp[b] : 0.f;
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(d, d);
  // the loads stay where they are written (the scheduler would otherwise
  // sink them next to their use and serialise the memory round trips)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NORMED) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < SSL; ++i) ss += ssv[i];
    if (sp)
      for (int b = rq + 8 * SSL; b < a.nss_in; b += 8) ss += sp[b];
    ss = group_sum<8>(ss);
    if (rq == 0) s_inv[rr] = a.ss_in ? 1.0f / sqrtf(ss / (float)a.hn + a.eps) : 1.f;
  }
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    const int d = t % DEPTH;
    // steps past the split end meet zero activations (a mask, so that the
    // step's MFMAs and the counter waits stay unconditional)
    const uint32_t mk = 0u - (uint32_t)(kb + (t * NWV + wave) * kDecKStep < ke);
    auto keep = [mk](uint4 v) { return make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk); };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Bf16x8 ah = as_bf16x8(keep(av[d][i][0])), al = as_bf16x8(keep(av[d][i][1]));
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const Bf16x8 b = as_bf16x8(wv[d][j]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[i][j], 0, 0, 0);
      }
    }
    if (t + DEPTH < NKS) issue(d, t + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the waves' tiles added in LDS (C layout: column 16 j + li, rows 16 i +
  // 4 lg + r): waves 4..7 store, waves 0..3 add theirs (tile w + tile w + 4)
  float* st = reinterpret_cast<float*>(&s_t[wave & 3][0][0]);
  if (wave >= 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(i * 16 + lg * 4 + r) * TC + j * 16 + li] = acc[i][j][r];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* p = st + (i * 16 + lg * 4 + r) * TC + j * 16 + li;
          *p = acc[i][j][r] + *p;
        }
  }
  __syncthreads();
  // item h of this thread: row er[h], column group c[h] (its columns 4 c ..
  // 4 c + 3; SwiGLU: gate columns 4 c .., up columns TC / 2 + 4 c ..)
  const bool act = tid < AT;
  int er[NH], cg[NH];
  float4 v[NH][NV];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int ii = min(h * NT + tid, IT - 1);
    er[h] = ii / TPR;
    cg[h] = ii % TPR;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c4 = (u ? TC / 8 : 0) + cg[h];
      float4 x = s_t[0][er[h]][c4];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 y = s_t[w][er[h]][c4];
        x = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
      }
      v[h][u] = x;
    }
  }

  if constexpr (EPI == kDecParts) {
    if (!act) return;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float* pp = a.part + ((size_t)split * kMmaRows + er[h]) * a.N;
      const int n = tile * TC + 4 * cg[h];
      if (n + 4 <= a.N) {
        *reinterpret_cast<float4*>(pp + n) = v[h][0];
      } else {
        const float f[4] = {v[h][0].x, v[h][0].y, v[h][0].z, v[h][0].w};
        for (int e = 0; e < 4 && n + e < a.N; ++e) pp[n + e] = f[e];
      }
    }
    return;
  } else {
    constexpr int TSZ = kMmaRows * TC;   // floats of one split's tile
    if (a.ks > 1) {
      // piece p (two floats) of thread tid at [tile, split, p, tid]: every
      // store (and load below) of a wave covers 512 contiguous bytes
      float* tp = a.part + ((size_t)tile * a.ks + split) * TSZ + tid * 2;
      if (act) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int u = 0; u < NV; ++u) {
            const int p = (h * NV + u) * 2;
            store_coherent2(tp + p * (2 * AT), v[h][u].x, v[h][u].y);
            store_coherent2(tp + (p + 1) * (2 * AT), v[h][u].z, v[h][u].w);
          }
      }
      __builtin_amdgcn_s_waitcnt(0);   // this thread's tile stores are complete
      __syncthreads();
      if (tid == 0) {
        int* t = a.ticket + tile;
        const int old = __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == a.ks - 1;
        if (last) __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
      }
      __syncthreads();
      if (!s_last) return;
    }
    if (!act) return;   // whole waves (AT is a multiple of 64)
    // the epilogue's operands (rows clamped below M: rows >= M are never
    // stored) are loaded ahead of the split tiles, in the same round trip
    float4 bb[NH], xo[NH], g[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int erc = min(er[h], a.M - 1);
      const int n = min(tile * TC + 4 * cg[h], a.N - 4);   // N is a multiple of 4
      if constexpr (EPI == kDecStore) {
        // segment ends are multiples of 4: a column group lies in one segment
        const int sg = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
        const int sb = sg == 0 ? 0 : (sg == 1 ? a.seg_end[0] : a.seg_end[1]);
        const float* bp = pick3(a.bias, sg);
        bb[h] = bp ? *reinterpret_cast<const float4*>(bp + (n - sb)) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else if constexpr (EPI == kDecResidual) {
        xo[h] = *reinterpret_cast<const float4*>(a.out + (size_t)erc * a.ldo + n);
        g[h] = *reinterpret_cast<const float4*>(a.gain + n);
      }
    }
    if (a.ks > 1) {
      // every split's tile, added in split order; up to NB splits' loads in
      // flight at once (indexes past the last split re-read it and are skipped)
      constexpr int NB = 8;
      const float* tb = a.part + (size_t)tile * a.ks * TSZ + tid * 2;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int u = 0; u < NV; ++u) v[h][u] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s0 = 0; s0 < a.ks; s0 += NB) {
        float4 w4[NB][NH][NV];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float* sp = tb + (size_t)min(s0 + b, a.ks - 1) * TSZ;
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int u = 0; u < NV; ++u) {
              const int p = (h * NV + u) * 2;
              load_coherent2(sp + p * (2 * AT), w4[b][h][u].x, w4[b][h][u].y);
              load_coherent2(sp + (p + 1) * (2 * AT), w4[b][h][u].z, w4[b][h][u].w);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (s0 + b < a.ks) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
              for (int u = 0; u < NV; ++u)
                v[h][u] = make_float4(v[h][u].x + w4[b][h][u].x, v[h][u].y + w4[b][h][u].y,
                                      v[h][u].z + w4[b][h][u].z, v[h][u].w + w4[b][h][u].w);
          }
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int row = er[h];
      const float inv = NORMED ? s_inv[row] : 1.f;
      if constexpr (EPI == kDecStore) {
        const int n = tile * TC + 4 * cg[h];
        if (row < a.M && n < a.N)
          *reinterpret_cast<float4*>(a.out + (size_t)row * a.ldo + n) =
              make_float4(v[h][0].x * inv + bb[h].x, v[h][0].y * inv + bb[h].y,
                          v[h][0].z * inv + bb[h].z, v[h][0].w * inv + bb[h].w);
      } else if constexpr (EPI == kDecResidual) {
        const int n = tile * TC + 4 * cg[h];
        float sq = 0.f;
        if (row < a.M && n < a.N) {
          const float4 t = make_float4(xo[h].x + v[h][0].x, xo[h].y + v[h][0].y,
                                       xo[h].z + v[h][0].z, xo[h].w + v[h][0].w);
          *reinterpret_cast<float4*>(a.out + (size_t)row * a.ldo + n) = t;
          const float xg[4] = {t.x * g[h].x, t.y * g[h].y, t.z * g[h].z, t.w * g[h].w};
          uint16_t hv[4], lv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_hi_lo(xg[e], hv[e], lv[e]);
          const size_t off = frag_off(row, n);
          *reinterpret_cast<uint2*>(a.ohi + off) =
              make_uint2(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16));
          *reinterpret_cast<uint2*>(a.olo + off) =
              make_uint2(lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16));
          sq = (t.x * t.x + t.y * t.y) + (t.z * t.z + t.w * t.w);
        }
        // kSsCols = 16 columns: four adjacent lanes (all active here)
        sq = group_sum<4>(sq);
        if ((cg[h] & 3) == 0 && row < a.M && n < a.N)
          a.ss_out[(size_t)row * ((a.N + kSsCols - 1) / kSsCols) + n / kSsCols] = sq;
      } else {   // kDecSwiglu
        const int F = a.N / 2;
        const int n = tile * (TC / 2) + 4 * cg[h];
        if (row < a.M && n < F) {   // F is a multiple of 4 (checked at launch)
          const float4 gv = v[h][0], uv = v[h][1];
          const float gg[4] = {gv.x * inv, gv.y * inv, gv.z * inv, gv.w * inv};
          const float uu[4] = {uv.x * inv, uv.y * inv, uv.z * inv, uv.w * inv};
          uint16_t hv[4], lv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_hi_lo(gg[e] / (1.0f + expf(-gg[e])) * uu[e], hv[e], lv[e]);
          const size_t off = frag_off(row, n);
          *reinterpret_cast<uint2*>(a.ohi + off) =
              make_uint2(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16));
          *reinterpret_cast<uint2*>(a.olo + off) =
              make_uint2(lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ generation bookkeeping
__global__ void k_record_token(const int32_t* tok, int32_t* out, int32_t* counter) {
  if (threadIdx.x == 0) {
    const int k = *counter;
    if (out) out[k] = *tok;
    *counter = k + 1;
  }
}

// one wave: every lane reads the counter before lane 0 moves it on
__global__ void k_record_tokens(const int32_t* src, int n, int32_t* out, int32_t* counter) {
  const int i = threadIdx.x;
  const int k = *counter;
  if (out && i < n) out[(size_t)k * n + i] = src[i];
  if (i == 0) *counter = k + 1;
}

__global__ void k_copy_f32(const float* src, float* dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ void k_fill_i32(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------ launchers

hipError_t launch_embed(const EmbedArgs& a, int bf16, hipStream_t s) {
  dim3 grid((a.h + 255) / 256, a.M);
  if (bf16)
    hipLaunchKernelGGL(k_embed<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_embed<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// K slices per block and 16-byte chunks per lane per slice, from K.
// (nk <= 1024 is guaranteed by the config limits, so ki <= 4.)
static void gemv_shape(int K, int vec, int& ks, int& ki) {
  const int nk = K / vec;
  ks = nk >= 256 ? 4 : (nk >= 128 ? 2 : 1);
  ki = ((nk + ks - 1) / ks + 63) / 64;
}

// rows per wave group: 4 when that still leaves >= 512 blocks
static int gemv_rw(int N, int ks) { return ks == 4 || N >= 512 * (4 / ks) * 4 ? 4 : ks; }

void gemv_block_rows(int N, int K, int wtype, int& br, size_t& row_bytes) {
  int vec, bytes;
  switch (wtype) {
    case kWBF16:
    case kWBF16NT: vec = WFmt<uint16_t>::N; bytes = WFmt<uint16_t>::BYTES; break;
    case kWQ8: vec = WFmt<WQ8>::N; bytes = WFmt<WQ8>::BYTES; break;
    case kWQ4: vec = WFmt<WQ4>::N; bytes = WFmt<WQ4>::BYTES; break;
    default: vec = WFmt<float>::N; bytes = WFmt<float>::BYTES; break;
  }
  int ks, ki;
  gemv_shape(K, vec, ks, ki);
  br = (4 / ks) * gemv_rw(N, ks);
  row_bytes = (size_t)(K / vec) * bytes;
}

template <typename WT, int MR, int EPI, bool NORM>
static void gemv_dispatch_shape(const GemvArgs& a, hipStream_t s) {
  int ks, ki;
  gemv_shape(a.K, WFmt<WT>::N, ks, ki);
  const int rw = gemv_rw(a.N, ks);
  const int br = (4 / ks) * rw;   // rows per block
  const dim3 grid((a.N + br - 1) / br), block(256);
#define ATD_GEMV(KS_, KI_, RW_) \
  hipLaunchKernelGGL((k_gemv<WT, MR, KS_, KI_, EPI, NORM, RW_>), grid, block, 0, s, a)
  if (ks == 4) {
    switch (ki) {
      case 1: ATD_GEMV(4, 1, 4); break;
      case 2: ATD_GEMV(4, 2, 4); break;
      case 3: ATD_GEMV(4, 3, 4); break;
      default: ATD_GEMV(4, 4, 4); break;
    }
  } else if (ks == 2) {
    if (rw == 4) {
      if (ki == 1) ATD_GEMV(2, 1, 4); else ATD_GEMV(2, 2, 4);
    } else {
      if (ki == 1) ATD_GEMV(2, 1, 2); else ATD_GEMV(2, 2, 2);
    }
  } else {
    if (rw == 4) {
      if (ki == 1) ATD_GEMV(1, 1, 4); else ATD_GEMV(1, 2, 4);
    } else {
      if (ki == 1) ATD_GEMV(1, 1, 1); else ATD_GEMV(1, 2, 1);
    }
  }
#undef ATD_GEMV
}

template <typename WT, int EPI, bool NORM>
static void gemv_dispatch_mr(const GemvArgs& a, hipStream_t s) {
  for (int c = 0; c < a.M; c += kGemvMaxRows) {
    GemvArgs b = a;
    b.M = a.M - c < kGemvMaxRows ? a.M - c : kGemvMaxRows;
    b.x = a.x + (size_t)c * a.ldx;
    b.out = a.out + (size_t)c * a.ldo;
    b.y_out = a.y_out ? a.y_out + (size_t)c * a.K : nullptr;
    if (b.M == 2)
      gemv_dispatch_shape<WT, 2, EPI, NORM>(b, s);
    else
      gemv_dispatch_shape<WT, 1, EPI, NORM>(b, s);
  }
}

template <typename WT>
static void gemv_dispatch(const GemvArgs& a, int epi, bool norm, hipStream_t s) {
  if (epi == kEpiStore && norm)
    gemv_dispatch_mr<WT, kEpiStore, true>(a, s);
  else if (epi == kEpiStore)
    gemv_dispatch_mr<WT, kEpiStore, false>(a, s);
  else if (epi == kEpiResidual)
    gemv_dispatch_mr<WT, kEpiResidual, false>(a, s);
  else
    gemv_dispatch_mr<WT, kEpiSwiglu, true>(a, s);
}

// ------------------------------------------------------------------ codec convolution GEMM
// One launch is a GEMM y[co][t] = sum_r W[co][r] X[r][t] over r = (input channel
// ci, tap j), X[r][t] = x[ci][t - (K-1-j) dil] (zero before frame 0), on the
// float32 matrix cores (v_mfma_f32_16x16x4f32: products and sums in float32).
// Phases (blockIdx.z = p < P) take their own weights [P][cout][R] and write
// y[co][t * ystride + p] (a transposed convolution by phase: K = 2 taps, the
// previous frame and this one).  Workgroup: 4 waves in 2 x 2, each wave
// (16 WM) channels x (16 WN) frames; the reduction runs in chunks of BK,
// staged in LDS, the next chunk's global loads held in registers while the
// MFMAs run on this one.  Within each 16 reduction indices an LDS row holds
// index k at (k % 4) * 4 + k / 4, so that a lane reads its four MFMA k-steps
// (k = 4s + lane / 16) as one float4.
template <int WM, int WN, int BK>
__global__ __launch_bounds__(256) void k_conv1d(ConvArgs a) {
  constexpr int BM = 32 * WM, BN = 32 * WN, LD = BK + 4;
  constexpr int AE = BM * BK / 256, BE = BN * BK / 256;   // elements per thread
  constexpr int AT = BK / AE;                               // threads per A row
  constexpr int BT = 256 / BK;                              // threads per B row
  static_assert(AE >= 1 && BE >= 1 && BK % 16 == 0, "tile shape");
  __shared__ __align__(16) float As[2][BM][LD];
  __shared__ __align__(16) float Bs[2][BN][LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.y * BM, t0 = blockIdx.x * BN, p = blockIdx.z;
  const int R = a.cin * a.K;
  const float* W = a.w + (size_t)p * a.cout * R;
  // A: thread -> channel row am, reduction indices ak .. ak + AE - 1 (contiguous in W)
  const int am = tid / AT, ak = (tid % AT) * AE;
  const bool arow = c0 + am < a.cout;
  const float* wr = W + (size_t)(arow ? c0 + am : 0) * R;
  // B: thread -> reduction index bk, frames bn .. bn + BE - 1 (contiguous in x)
  const int bk = tid / BT, bn = (tid % BT) * BE;
  const int bkp = (bk & ~15) | ((bk & 3) * 4 + ((bk & 15) >> 2));
  float ra[AE], rb[BE];
  // weight rows in 16-byte pieces when every row start is 16-byte aligned
  const bool avec = (AE % 4 == 0) && (R % 4 == 0) && (((uintptr_t)W & 15) == 0);
  // input rows likewise when T % 4 == 0 (frame groups of 4 never straddle 0 or T)
  const bool bvec = (BE % 4 == 0) && (a.T % 4 == 0) && (((uintptr_t)a.x & 15) == 0);
  auto load = [&](int r0) {
    if (avec) {
#pragma unroll
      for (int e = 0; e < AE; e += 4) {
        const int r = r0 + ak + e;
        const float4 v = (arow && r < R) ? *reinterpret_cast<const float4*>(wr + r)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
        ra[e] = v.x;
        ra[e + 1] = v.y;
        ra[e + 2] = v.z;
        ra[e + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < AE; ++e) {
        const int r = r0 + ak + e;
        ra[e] = (arow && r < R) ? wr[r] : 0.f;
      }
    }
    const int r = r0 + bk;
    const int ci = r / a.K, j = r - ci * a.K;
    const int t = t0 + bn - (a.K - 1 - j) * a.dil;
    const float* xr = a.x + (size_t)(r < R ? ci : 0) * a.T;
    if (bvec) {
      // the BE frames from BE / 4 + 1 aligned 16-byte pieces (each wholly
      // inside or outside [0, T), as T % 4 == 0), then shifted by t % 4
      const int tb = t & ~3, m = t & 3;
      float v[BE + 4];
#pragma unroll
      for (int q = 0; q < BE / 4 + 1; ++q) {
        const int tq = tb + 4 * q;
        const float4 f = (r < R && tq >= 0 && tq < a.T)
                             ? *reinterpret_cast<const float4*>(xr + tq)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
      switch (m) {   // constant register indices in every branch
        case 0:
#pragma unroll
          for (int e = 0; e < BE; ++e) rb[e] = v[e];
          break;
        case 1:
#pragma unroll
          for (int e = 0; e < BE; ++e) rb[e] = v[e + 1];
          break;
        case 2:
#pragma unroll
          for (int e = 0; e < BE; ++e) rb[e] = v[e + 2];
          break;
        default:
#pragma unroll
          for (int e = 0; e < BE; ++e) rb[e] = v[e + 3];
          break;
      }
    } else {
#pragma unroll
      for (int e = 0; e < BE; ++e)
        rb[e] = (r < R && t + e >= 0 && t + e < a.T) ? xr[t + e] : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < AE; ++e) {
      const int k = ak + e;
      As[buf][am][(k & ~15) | ((k & 3) * 4 + ((k & 15) >> 2))] = ra[e];
    }
#pragma unroll
    for (int e = 0; e < BE; ++e) Bs[buf][bn + e][bkp] = rb[e];
  };
  Floatx4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int k = 0; k < WN; ++k) acc[i][k] = Floatx4{0.f, 0.f, 0.f, 0.f};
  const int wm0 = (wave >> 1) * 16 * WM, wn0 = (wave & 1) * 16 * WN;
  const int lr = lane & 15, lq = (lane >> 4) * 4;
  const int nchunk = (R + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunk) load((c + 1) * BK);
#pragma unroll
    for (int g = 0; g < BK; g += 16) {
      float4 fa[WM], fb[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        fa[i] = *reinterpret_cast<const float4*>(&As[buf][wm0 + 16 * i + lr][g + lq]);
#pragma unroll
      for (int k = 0; k < WN; ++k)
        fb[k] = *reinterpret_cast<const float4*>(&Bs[buf][wn0 + 16 * k + lr][g + lq]);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int k = 0; k < WN; ++k) {
          acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i].x, fb[k].x, acc[i][k], 0, 0, 0);
          acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i].y, fb[k].y, acc[i][k], 0, 0, 0);
          acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i].z, fb[k].z, acc[i][k], 0, 0, 0);
          acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i].w, fb[k].w, acc[i][k], 0, 0, 0);
        }
    }
    if (c + 1 < nchunk) store(buf ^ 1);
    __syncthreads();
  }
  // lane holds rows 4 (lane / 16) + e, column lane % 16 of each 16 x 16 block
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int co = c0 + wm0 + 16 * i + lq + e;
      if (co >= a.cout) continue;
      const float bv = a.bias ? a.bias[co] : 0.f;
      float* yr = a.y + (size_t)co * a.ldy + p;
#pragma unroll
      for (int k = 0; k < WN; ++k) {
        const int t = t0 + wn0 + 16 * k + lr;
        if (t < a.T) {
          float* o = yr + (size_t)t * a.ystride;
          *o = (a.accumulate ? *o : 0.f) + (acc[i][k][e] + bv);
        }
      }
    }
}

template <int WM, int WN, int BK>
void conv_launch(const ConvArgs& a, hipStream_t s) {
  const dim3 g((a.T + 32 * WN - 1) / (32 * WN), (a.cout + 32 * WM - 1) / (32 * WM), a.P);
  hipLaunchKernelGGL((k_conv1d<WM, WN, BK>), g, dim3(256), 0, s, a);
}

// ------------------------------------------------------------------ prefill attention
// Causal attention of a prefill chunk's rows on the float32 matrix cores
// (v_mfma_f32_16x16x4f32), flash style.  Workgroup = 16 query rows x HP query
// heads of one KV head x KS key lanes: wave (head j, key lane kp) takes keys
// kp*32 .. kp*32+31 of every staged tile of KS*32 keys, with its own running
// max / sum / output; the KS partial states of a head are merged at the end.
// Tiles are staged once in LDS (float32) for all waves, the next tile's loads
// in flight while the current one is computed.  Per 32 keys a wave forms
// S = Q K^T (16 x 32), masks keys past each row's position, updates the
// running max / sum, writes P through LDS to reach the A layout and
// accumulates O += P V.  The contraction order over channels (and over keys
// in P V) is permuted so that a lane's Q, K and P operands of four
// successive MFMA k-steps are four adjacent floats, read with one 16-byte LDS
// load (V, the B operand of P V, is read per k-step): k-step 4j + t of lane
// group lg takes index 16j + 4lg + t.
template <typename KT, int D, int HP, int KS>
__global__ __launch_bounds__(64 * HP * KS) void k_attn_prefill(AttnArgs a) {
  constexpr int NW = HP * KS;          // waves
  constexpr int NT = 64 * NW;          // threads
  constexpr int KI = 32 * KS;          // keys staged per iteration
  constexpr int DS = D + 4;            // LDS row stride (16-byte aligned)
  constexpr int NB = D / 16;           // 16-column blocks of O
  constexpr int VEC = Vec16<KT>::N;
  constexpr int PER = KI * D / VEC / NT;   // 16-byte loads per thread per matrix
  static_assert(PER * VEC * NT == KI * D, "tile does not divide over the threads");
  __shared__ __align__(16) float Ks[KI * DS];
  __shared__ __align__(16) float Vs[KI * DS];
  __shared__ __align__(16) float Ps[NW][16 * 36];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int jh = wave % HP, kp = wave / HP;
  const int R = a.Hq / a.Hkv, groups = R / HP;
  const int g = blockIdx.y / groups;
  const int h = g * R + (blockIdx.y % groups) * HP + jh;
  const int m0 = (gridDim.x - 1 - blockIdx.x) * 16;   // longest key ranges first
  const int p0 = a.rows.row0;                          // position of the launch's row 0
  const int kmax = p0 + min(m0 + 16, a.M);             // keys the rows read
  const KT* Kh = reinterpret_cast<const KT*>(a.k_direct) + (size_t)g * a.cap_direct * D;
  const KT* Vh = reinterpret_cast<const KT*>(a.v_direct) + (size_t)g * a.cap_direct * D;

  // queries as A operands (row m0 + li), pre-scaled by 1/sqrt(D)
  float qf[D / 4];
  {
    const float* qp = a.q + ((size_t)min(m0 + li, a.M - 1) * a.Hq + h) * D;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(qp + 16 * j + 4 * lg);
      qf[4 * j] = v.x * a.scale;
      qf[4 * j + 1] = v.y * a.scale;
      qf[4 * j + 2] = v.z * a.scale;
      qf[4 * j + 3] = v.w * a.scale;
    }
  }
  Floatx4 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = Floatx4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrow[i] = -1e30f;
    lrow[i] = 0.f;
  }

  // tile loads (key rows clamped into the valid range; the rows past kmax
  // are masked below)
  uint4 kr[PER], vr[PER];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + e * NT;
      const int r = idx / (D / VEC), c = (idx % (D / VEC)) * VEC;
      const int key = min(k0 + r, kmax - 1);
      kr[e] = ldg16(Kh + (size_t)key * D + c);
      vr[e] = ldg16(Vh + (size_t)key * D + c);
    }
  };
  const int nit = (kmax + KI - 1) / KI;
  load_tile(0);
  for (int it = 0; it < nit; ++it) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + e * NT;
      const int r = idx / (D / VEC), c = (idx % (D / VEC)) * VEC;
      float kv[VEC], vv[VEC];
      Vec16<KT>::unpack(kr[e], kv);
      Vec16<KT>::unpack(vr[e], vv);
#pragma unroll
      for (int t = 0; t < VEC; t += 4) {
        *reinterpret_cast<float4*>(&Ks[r * DS + c + t]) =
            make_float4(kv[t], kv[t + 1], kv[t + 2], kv[t + 3]);
        *reinterpret_cast<float4*>(&Vs[r * DS + c + t]) =
            make_float4(vv[t], vv[t + 1], vv[t + 2], vv[t + 3]);
      }
    }
    __syncthreads();
    load_tile((it + 1) * KI);   // next tile in flight during the math
    const int kb0 = it * KI + kp * 32;   // first key of this wave's 32
    const float* Kw = Ks + kp * 32 * DS;
    const float* Vw = Vs + kp * 32 * DS;
    // S = Q K^T for two 16-key blocks
    Floatx4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = Floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 kf = *reinterpret_cast<const float4*>(Kw + (kb * 16 + li) * DS + 16 * j + 4 * lg);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * j], kf.x, sc[kb], 0, 0, 0);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * j + 1], kf.y, sc[kb], 0, 0, 0);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * j + 2], kf.z, sc[kb], 0, 0, 0);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * j + 3], kf.w, sc[kb], 0, 0, 0);
      }
    }
    // lane holds rows m0 + 4 lg + i, keys kb0 + 16 kb + li
    float* Pw = Ps[wave];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = p0 + m0 + 4 * lg + i;
      float s0 = sc[0][i], s1 = sc[1][i];
      if (kb0 + li > pos) s0 = -1e30f;
      if (kb0 + 16 + li > pos) s1 = -1e30f;
      float tm = fmaxf(s0, s1);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) tm = fmaxf(tm, __shfl_xor(tm, off, 64));
      const float mn = fmaxf(mrow[i], tm);
      const float c = expf(mrow[i] - mn);
      const float e0 = expf(s0 - mn), e1 = expf(s1 - mn);
      float ts = e0 + e1;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ts += __shfl_xor(ts, off, 64);
      lrow[i] = lrow[i] * c + ts;
      mrow[i] = mn;
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b][i] *= c;
      Pw[(4 * lg + i) * 36 + li] = e0;
      Pw[(4 * lg + i) * 36 + 16 + li] = e1;
    }
    // P is read back by other lanes of the same wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O += P V
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 pa = *reinterpret_cast<const float4*>(Pw + li * 36 + 16 * j + 4 * lg);
      const float* vrow = Vw + (16 * j + 4 * lg) * DS + li;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        o[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa.x, vrow[16 * b], o[b], 0, 0, 0);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa.y, vrow[DS + 16 * b], o[b], 0, 0, 0);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa.z, vrow[2 * DS + 16 * b], o[b], 0, 0, 0);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa.w, vrow[3 * DS + 16 * b], o[b], 0, 0, 0);
      }
    }
    __syncthreads();   // the tile buffers are refilled next
  }
  // merge the key lanes of a head: lanes kp > 0 leave (max, sum, O) in LDS
  // (the K buffer, free after the last barrier), key lane 0 combines
  if (KS > 1) {
    static_assert(KS == 1 || (KS - 1) * HP * 16 * (D + 2) <= KI * DS, "merge area");
    if (kp > 0) {
      float* mg = Ks + ((kp - 1) * HP + jh) * 16 * (D + 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        if (li == 0) {
          mg[r * (D + 2) + D] = mrow[i];
          mg[r * (D + 2) + D + 1] = lrow[i];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) mg[r * (D + 2) + 16 * b + li] = o[b][i];
      }
    }
    __syncthreads();
    if (kp > 0) return;
#pragma unroll
    for (int q = 1; q < KS; ++q) {
      const float* mg = Ks + ((q - 1) * HP + jh) * 16 * (D + 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        const float m2 = mg[r * (D + 2) + D], l2 = mg[r * (D + 2) + D + 1];
        const float mn = fmaxf(mrow[i], m2);
        const float c1 = expf(mrow[i] - mn), c2 = expf(m2 - mn);
        lrow[i] = lrow[i] * c1 + l2 * c2;
        mrow[i] = mn;
#pragma unroll
        for (int b = 0; b < NB; ++b) o[b][i] = o[b][i] * c1 + mg[r * (D + 2) + 16 * b + li] * c2;
      }
    }
  }
  // rows m0 + 4 lg + i, channels 16 b + li
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * lg + i;
    if (m >= a.M) continue;
    const float inv = 1.0f / lrow[i];
    const size_t off = ((size_t)m * a.Hq + h) * D;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = o[b][i] * inv;
      if (a.o_hi) {
        uint16_t hv, lv;
        split_hi_lo(v, hv, lv);
        const size_t oo = a.o_frag ? frag_off(m, h * D + 16 * b + li) : off + 16 * b + li;
        a.o_hi[oo] = hv;
        a.o_lo[oo] = lv;
      } else {
        a.o[off + 16 * b + li] = v;
      }
    }
  }
}

// heads per workgroup and key lanes by group size: 1 -> 1 x 4 (four waves),
// 2 -> 2 x 4, 4 and 8 -> 4 x 2 (eight waves; 8: two workgroups per KV head).
// Two waves per SIMD hide the latency of each wave's serial tile walk
// (measured at 512 rows of the 1.7B shape: 2 x 2 key lanes 46.6 us per
// layer, 2 x 4 lanes 36.9 us)
template <typename KT, int D>
static void attn_prefill_r(const AttnArgs& a, int r, hipStream_t s) {
  const int hp = r < 4 ? r : 4;
  const dim3 grid((a.M + 15) / 16, a.Hkv * (r / hp));
  if (r == 1)
    hipLaunchKernelGGL((k_attn_prefill<KT, D, 1, 4>), grid, dim3(256), 0, s, a);
  else if (r == 2)
    hipLaunchKernelGGL((k_attn_prefill<KT, D, 2, 4>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_prefill<KT, D, 4, 2>), grid, dim3(512), 0, s, a);
}

hipError_t launch_attn_prefill(const AttnArgs& a, int bf16, int D, int r, hipStream_t s) {
  if (a.fused || a.rows.mode != kRowsPrefill || !a.k_direct || a.M < 1 ||
      (r != 1 && r != 2 && r != 4 && r != 8) || a.Hq != a.Hkv * r)
    return hipErrorInvalidValue;
  if (bf16) {
    if (D == 64) attn_prefill_r<uint16_t, 64>(a, r, s);
    else attn_prefill_r<uint16_t, 128>(a, r, s);
  } else {
    if (D == 64) attn_prefill_r<float, 64>(a, r, s);
    else attn_prefill_r<float, 128>(a, r, s);
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a, int epi, bool norm, int wtype, hipStream_t s) {
  switch (wtype) {
    case kWBF16: gemv_dispatch<uint16_t>(a, epi, norm, s); break;
    case kWBF16NT: gemv_dispatch<Bf16Nt>(a, epi, norm, s); break;
    case kWQ8: gemv_dispatch<WQ8>(a, epi, norm, s); break;
    case kWQ4: gemv_dispatch<WQ4>(a, epi, norm, s); break;
    default: gemv_dispatch<float>(a, epi, norm, s); break;
  }
  return hipGetLastError();
}

// Tile of a convolution GEMM (measured over the codec decoder's layer shapes):
// 64 x 64 while that grid gives ~3 workgroups per compute unit, then 64 x 32
// with a deeper reduction chunk, then 32 x 32; 32 x 64 for <= 32 output
// channels, where a 64-channel tile would be mostly idle.
hipError_t launch_conv(const ConvArgs& a, hipStream_t s) {
  auto blocks = [&](int bm, int bn) {
    return (long)((a.T + bn - 1) / bn) * ((a.cout + bm - 1) / bm) * a.P;
  };
  if (a.cout <= 32) conv_launch<1, 2, 64>(a, s);
  else if (blocks(64, 64) >= 700) conv_launch<2, 2, 32>(a, s);
  else if (blocks(64, 32) >= 400) conv_launch<2, 1, 64>(a, s);
  else conv_launch<1, 1, 64>(a, s);
  return hipGetLastError();
}

hipError_t launch_pack_transconv(const float* w, int cin, int cout, int s_, float* packed,
                                 hipStream_t s) {
  const size_t n = (size_t)s_ * cout * cin * 2;
  const size_t nb = (n + 255) / 256;
  const unsigned blocks = (unsigned)(nb < 65535 ? nb : 65535);
  hipLaunchKernelGGL(k_pack_transconv, dim3(blocks), dim3(256), 0, s, w, cin, cout, s_, packed);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t blocks = a.rows * (a.cols / kQBlock);
  const dim3 grid((unsigned)((blocks + 255) / 256)), block(256);
  if (a.bf16) {
    if (a.q4) hipLaunchKernelGGL((k_quantize<uint16_t, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_quantize<uint16_t, false>), grid, block, 0, s, a);
  } else {
    if (a.q4) hipLaunchKernelGGL((k_quantize<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_quantize<float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeArgs& a, int bf16, hipStream_t s) {
  if ((a.D != 64 && a.D != 128) || a.M < 1) return hipErrorInvalidValue;
  const long items = (long)a.M * (a.Hq + 2 * a.Hkv);
  const int per_block = 4 * (128 / a.D);   // waves x items per wave
  const dim3 grid((unsigned)((items + per_block - 1) / per_block));
  if (a.D == 64) {
    if (bf16) hipLaunchKernelGGL((k_rope_append<uint16_t, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_rope_append<float, 64>), grid, dim3(256), 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((k_rope_append<uint16_t, 128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_rope_append<float, 128>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <typename KT, int D>
static void attn_dispatch_r(const AttnArgs& a, int r, dim3 grid, hipStream_t s) {
  // lanes per key row and rows per lane group per tile (measured on the
  // 1.7B shape: a bf16 cache row of 128 channels is best read by 8 lanes, a
  // float32 row by 16)
  constexpr int LPK0 = sizeof(KT) == 2 ? 8 : 16;
  constexpr int LPK = LPK0 < D / Vec16<KT>::N ? LPK0 : D / Vec16<KT>::N;
  constexpr int U = 2;
  const dim3 mgrid(a.Hkv, a.M);
  if (a.defer) {
    switch (r) {
      case 1: hipLaunchKernelGGL((k_attn_split<KT, D, 1, LPK, U, true>), grid, dim3(256), 0, s, a);
              hipLaunchKernelGGL((k_attn_merge<D, 1>), mgrid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((k_attn_split<KT, D, 2, LPK, U, true>), grid, dim3(256), 0, s, a);
              hipLaunchKernelGGL((k_attn_merge<D, 2>), mgrid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((k_attn_split<KT, D, 4, LPK, U, true>), grid, dim3(256), 0, s, a);
              hipLaunchKernelGGL((k_attn_merge<D, 4>), mgrid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((k_attn_split<KT, D, 8, LPK, U, true>), grid, dim3(256), 0, s, a);
               hipLaunchKernelGGL((k_attn_merge<D, 8>), mgrid, dim3(256), 0, s, a); break;
    }
    return;
  }
  switch (r) {
    case 1: hipLaunchKernelGGL((k_attn_split<KT, D, 1, LPK, U, false>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn_split<KT, D, 2, LPK, U, false>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn_split<KT, D, 4, LPK, U, false>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_attn_split<KT, D, 8, LPK, U, false>), grid, dim3(256), 0, s, a); break;
  }
}

hipError_t launch_attention(const AttnArgs& a, int bf16, int D, int r, hipStream_t s) {
  if (a.pf.nreg < 0 || a.pf.nreg > kPfRegions || (a.defer && a.pf.nreg)) return hipErrorInvalidValue;
  for (int i = 0; i < a.pf.nreg; ++i)
    if (!a.pf.base[i] || a.pf.bb[i] % 16 || a.pf.nblk[i] < 0) return hipErrorInvalidValue;
  dim3 grid((a.nsplit_max + 3) / 4, a.Hkv, a.M + (a.pf.nreg > 0 ? 1 : 0));
  if (bf16) {
    if (D == 64)
      attn_dispatch_r<uint16_t, 64>(a, r, grid, s);
    else
      attn_dispatch_r<uint16_t, 128>(a, r, grid, s);
  } else {
    if (D == 64)
      attn_dispatch_r<float, 64>(a, r, grid, s);
    else
      attn_dispatch_r<float, 128>(a, r, grid, s);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void k_mrope_rows(const int32_t* pos3, int half, int sec_h,
                                                   int sec_w, int max_ctx, const float* cos_t,
                                                   const float* sin_t, float* rcos, float* rsin) {
  const int m = blockIdx.x, i = threadIdx.x;
  if (i >= half) return;
  const int r = i % 3;
  const int c = (r == 1 && i < 3 * sec_h) ? 1 : ((r == 2 && i < 3 * sec_w) ? 2 : 0);
  int p = pos3[m * 3 + c];
  p = p < 0 ? 0 : (p >= max_ctx ? max_ctx - 1 : p);
  rcos[(size_t)m * half + i] = cos_t[(size_t)p * half + i];
  rsin[(size_t)m * half + i] = sin_t[(size_t)p * half + i];
}

hipError_t launch_mrope_rows(const int32_t* pos3, int M, int half, int sec_h, int sec_w,
                             int max_ctx, const float* cos_t, const float* sin_t, float* rcos,
                             float* rsin, hipStream_t s) {
  if (M < 1 || half > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mrope_rows, dim3(M), dim3(64), 0, s, pos3, half, sec_h, sec_w, max_ctx,
                     cos_t, sin_t, rcos, rsin);
  return hipGetLastError();
}

// Streaming read of n16 16-byte chunks (measurement of the attainable read
// bandwidth): every block reads 8 chunks per thread per pass (32 KB), the
// grid strides over the buffer; the loaded words are folded into one value
// that is stored only if it equals a constant, so the loads are kept.
__global__ __launch_bounds__(256) void k_read_stream(const uint4* p, size_t n16, uint32_t* sink) {
  constexpr int U = 8;
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t base = (size_t)blockIdx.x * 256 * U; base < n16; base += stride) {
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * 256 + tid;
      r[u] = ldg16(p + (i < n16 ? i : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t per_block = 256 * 8;
  size_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 4096) blocks = 4096;   // 16 per compute unit; the grid strides over the rest
  hipLaunchKernelGGL(k_read_stream, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_advance(const SlotTables& st, RowMap rows, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_advance, dim3((M + 255) / 256), dim3(256), 0, s, st, rows, M);
  return hipGetLastError();
}

hipError_t launch_slot_list(int32_t* dst, const int32_t* slots, int n, hipStream_t s) {
  for (int off = 0; off < n; off += kSlotListChunk) {
    SlotListArgs a{};
    a.n = n - off < kSlotListChunk ? n - off : kSlotListChunk;
    a.off = off;
    for (int i = 0; i < a.n; ++i) a.v[i] = slots[off + i];
    hipLaunchKernelGGL(k_slot_list, dim3(1), dim3(kSlotListChunk), 0, s, dst, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_set_slot(const SlotTables& st, int slot, void* const* k, void* const* v,
                           int cap, int pos, int set_ptrs, hipStream_t s) {
  SlotSetArgs a{};
  a.slot = slot;
  a.cap = cap;
  a.pos = pos;
  a.set_ptrs = set_ptrs;
  if (set_ptrs)
    for (int l = 0; l < st.L; ++l) {
      a.k[l] = k[l];
      a.v[l] = v[l];
    }
  hipLaunchKernelGGL(k_set_slot, dim3(1), dim3(64), 0, s, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_copy(const KvCopyArgs& a, hipStream_t s) {
  const size_t n16 = (size_t)a.rows * a.D * a.elem_bytes / 16;
  int bx = (int)((n16 + 255) / 256);
  if (bx > 64) bx = 64;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(k_kv_copy, dim3(bx, a.Hkv, a.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_argmax(const ArgmaxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_part, dim3(a.nblk, a.B), dim3(256), 0, s, a);
  if (a.nblk > 1) hipLaunchKernelGGL(k_argmax_final, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Partials of greedy_argmax_noalloc: a file-scope device array, so the call
// needs no allocation (each GPU the library runs on holds its own copy until
// the process ends).  In host code `scratch` only stands for the symbol; the
// array's address on a device is taken once with hipGetSymbolAddress while
// that device is current, and only that address is handed to kernels.
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

hipError_t noalloc_scratch(float** out) {
  static std::mutex mu;
  static float* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<float*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  if (a.nblk > 1)
    hipLaunchKernelGGL(k_sample_part, dim3(a.nblk, a.B), dim3(kSampleThreads), 0, s, a);
  hipLaunchKernelGGL(k_sample_final, dim3(a.B), dim3(kSampleThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_record_token(const int32_t* tok, int32_t* out, int32_t* counter,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_record_token, dim3(1), dim3(64), 0, s, tok, out, counter);
  return hipGetLastError();
}

hipError_t launch_record_tokens(const int32_t* src, int n, int32_t* out, int32_t* counter,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_record_tokens, dim3(1), dim3(64), 0, s, src, n, out, counter);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_f32, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.mrows < kMmaRows || a.mrows % kMmaRows) return hipErrorInvalidValue;
  const dim3 grid((a.N + kMmaBlockN - 1) / kMmaBlockN, a.ks, a.mrows / kMmaRows);
  // stages of a split (the last split may hold fewer real ones: the rest
  // read zero activations)
  switch ((a.kc + kMmaCh - 1) / kMmaCh) {
    case 1: hipLaunchKernelGGL((k_gemm<2, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<2, 2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_gemm<2, 3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_gemm<2, 4>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_gemm<2, 6>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_gemm<2, 8>), grid, dim3(256), 0, s, a); break;
    case 12: hipLaunchKernelGGL((k_gemm<2, 12>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_gemm<2, 16>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm<2, 0>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_tile(const GemmArgs& a, hipStream_t s) {
  if (a.mrows < kMmaRows || a.mrows % kMmaRows || a.K % 32 || a.kc % 32 || a.ks < 1 ||
      (long)a.kc * (a.ks - 1) >= a.K)
    return hipErrorInvalidValue;
  const dim3 grid((a.N + 127) / 128 * a.ks * ((a.mrows + 127) / 128));
  // 32-wide stages of a split (the last split may hold fewer real ones)
  switch (a.kc / 32) {
    case 2: hipLaunchKernelGGL(k_gemm_tile<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_gemm_tile<4>, grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL(k_gemm_tile<6>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_gemm_tile<8>, grid, dim3(256), 0, s, a); break;
    case 12: hipLaunchKernelGGL(k_gemm_tile<12>, grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL(k_gemm_tile<16>, grid, dim3(256), 0, s, a); break;
    case 24: hipLaunchKernelGGL(k_gemm_tile<24>, grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL(k_gemm_tile<32>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_gemm_tile<0>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int epi, hipStream_t s) {
  const int no = epi == kRedSwiglu ? a.N / 2 : a.N;
  // 4 columns per thread when every row, segment and output offset keeps
  // 16-byte alignment (a ragged vocabulary takes the scalar form) and the
  // grid still has >= 1024 blocks: measured at 512 prefill rows of the 1.7B
  // shape, 6.64 -> 6.41 ms per prefill; at 64 decode rows the 4x smaller
  // grid made the (latency-bound) reductions slower (12.24 k -> 12.16 k
  // tokens/s), so they keep one column per thread
  const bool vec4 = no % 4 == 0 && a.N % 4 == 0 && a.ldo % 4 == 0 && a.seg_end[0] % 4 == 0 &&
                    a.seg_end[1] % 4 == 0 && (long)((no + 1023) / 1024) * a.M >= 1024;
  if (vec4) {
    const dim3 grid4((no + 1023) / 1024, a.M);
    if (epi == kRedStore)
      hipLaunchKernelGGL(k_reduce4<kRedStore>, grid4, dim3(256), 0, s, a);
    else if (epi == kRedResidual)
      hipLaunchKernelGGL(k_reduce4<kRedResidual>, grid4, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_reduce4<kRedSwiglu>, grid4, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((no + 255) / 256, a.M);
  if (epi == kRedStore)
    hipLaunchKernelGGL(k_reduce<kRedStore>, grid, dim3(256), 0, s, a);
  else if (epi == kRedResidual)
    hipLaunchKernelGGL(k_reduce<kRedResidual>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_reduce<kRedSwiglu>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int EPI, int CB>
static void gemm_dec_dispatch(const DecGemmArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(64 * kDecWaves);
  switch (a.kc / (kDecWaves * kDecKStep)) {
    case 1: hipLaunchKernelGGL((k_gemm_dec<1, EPI, CB>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_gemm_dec<2, EPI, CB>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_gemm_dec<3, EPI, CB>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_gemm_dec<4, EPI, CB>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_gemm_dec<6, EPI, CB>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_gemm_dec<8, EPI, CB>), grid, block, 0, s, a); break;
    case 12: hipLaunchKernelGGL((k_gemm_dec<12, EPI, CB>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_dec<16, EPI, CB>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_swizzle_b(const SwizzleArgs& a, hipStream_t s) {
  if (a.K < 32 || a.K % 32 || a.N < 1 || (a.swiglu && a.N % 2) || !a.dst) return hipErrorInvalidValue;
  const size_t chunks = bfrag_blocks(a.N, a.swiglu != 0) * (a.K / 32) * 64;
  hipLaunchKernelGGL(k_swizzle_b, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_dec(const DecGemmArgs& a, int epi, hipStream_t s) {
  const int span = kDecWaves * kDecKStep;
  const int nks = a.kc / span;
  const bool nks_ok = nks >= 1 && nks <= kDecMaxSteps && (nks <= 4 || nks % 2 == 0) &&
                      (nks <= 8 || nks % 4 == 0);
  if (a.K < kDecKStep || a.K % kDecKStep || a.kc % span || !nks_ok || a.ks < 1 ||
      (long)a.kc * (a.ks - 1) >= a.K || (long)a.kc * a.ks < a.K || a.N < 4 || a.M < 1 ||
      a.M > kMmaRows || a.cb != dec_cb(epi, a.K) || !a.Wb ||
      (size_t)a.nblk != bfrag_blocks(a.N, epi == kDecSwiglu))
    return hipErrorInvalidValue;
  if (epi != kDecParts && (a.N % 4 || a.seg_end[0] % 4 || a.seg_end[1] % 4 || !a.ticket))
    return hipErrorInvalidValue;
  if (epi == kDecSwiglu && (a.N / 2) % 4) return hipErrorInvalidValue;
  const dim3 grid(dec_tiles(a.N, epi, a.K), a.ks);
  switch (epi * 8 + a.cb) {
    case kDecParts * 8 + 4: gemm_dec_dispatch<kDecParts, 4>(a, grid, s); break;
    case kDecStore * 8 + 1: gemm_dec_dispatch<kDecStore, 1>(a, grid, s); break;
    case kDecResidual * 8 + 1: gemm_dec_dispatch<kDecResidual, 1>(a, grid, s); break;
    case kDecResidual * 8 + 4: gemm_dec_dispatch<kDecResidual, 4>(a, grid, s); break;
    case kDecSwiglu * 8 + 4: gemm_dec_dispatch<kDecSwiglu, 4>(a, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace atd
