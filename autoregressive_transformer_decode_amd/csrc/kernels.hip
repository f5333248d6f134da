// HIP kernels of the decode step for gfx950 (CDNA4, wave64).
//
// The step of one layer follows the per-layer sequence profiled in the
// qwen3-tts-hip OPTIMIZATION_LOG (DecodeStepStack entry): input norm, q/k/v
// projection, q/k layout + cache write, attention, output projection +
// residual, post norm, gate/up projection, SwiGLU, down projection +
// residual.  Here the norms are fused into the projection that consumes
// them, SwiGLU into the gate/up projection, the residual adds into the
// projections that produce them, and no layout permute exists at all (the
// cache row is written in its final [Hkv, S, D] place).
//
// Decode at batch 1 is bound by HBM bandwidth: every weight byte is read
// once per step and used for one multiply-add per row.  The projections are
// therefore GEMVs that stream 16-byte vectors of weights per lane with all
// 64 lanes of a wave on consecutive addresses of one row, several rows per
// wave for bytes in flight, and the normalised input vector staged once per
// workgroup in LDS.  No matrix-core (MFMA) work is involved at this size.
//
// Attention at decode reads the K and V rows once; the key range is split
// into fixed chunks (split-K over the sequence) whose partial softmax
// states (running max, sum, weighted V) are merged in a fixed order, so
// results do not depend on the cache capacity or on launch timing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace atd {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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

__device__ __forceinline__ void row_of(const RowMap& r, const SlotTables& st, int m,
                                       int& slot, int& pos) {
  if (r.mode == kRowsPrefill) {
    slot = r.slot0;
    pos = m;
  } else {
    slot = r.slot0 + m;
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
  if (a.extra) s += a.extra[(size_t)m * a.h + i];
  a.out[(size_t)m * a.h + i] = s;
}

// ------------------------------------------------------------------ GEMV
// out[m, n] = epi( sum_k W[n, k] * xin[m, k] ),  xin = x or RMSNorm(x) * gain
// One wave owns RPW consecutive rows and sweeps k with 16-byte loads per
// lane; the (normalised) input rows sit in LDS.  MR input rows share every
// weight load.
template <typename WT, int MR, int RPW, int EPI, bool NORM>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];
  __shared__ float red[4][MR];
  constexpr int VEC = Vec16<WT>::N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;

  float ss[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    ss[m] = 0.f;
    const float* xr = a.x + (size_t)m * a.ldx;
    for (int i = tid * 4; i < K; i += 1024) {
      float4 v = *reinterpret_cast<const float4*>(xr + i);
      *reinterpret_cast<float4*>(xs + m * K + i) = v;
      ss[m] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float v = wave_sum(ss[m]);
      if (lane == 0) red[wave][m] = v;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float tot = red[0][m] + red[1][m] + red[2][m] + red[3][m];
      const float inv = 1.0f / sqrtf(tot / (float)K + a.eps);
      for (int i = tid * 4; i < K; i += 1024) {
        float4 v = *reinterpret_cast<float4*>(xs + m * K + i);
        const float4 g = *reinterpret_cast<const float4*>(a.gain + i);
        v.x = v.x * inv * g.x;
        v.y = v.y * inv * g.y;
        v.z = v.z * inv * g.z;
        v.w = v.w * inv * g.w;
        *reinterpret_cast<float4*>(xs + m * K + i) = v;
        if (a.y_out && blockIdx.x == 0)
          *reinterpret_cast<float4*>(a.y_out + (size_t)m * K + i) = v;
      }
    }
  }
  __syncthreads();

  const int row0 = (blockIdx.x * 4 + wave) * RPW;
  if (row0 >= a.N) return;
  const int s = row0 < a.seg_end[0] ? 0 : (row0 < a.seg_end[1] ? 1 : 2);
  const int sbeg = s == 0 ? 0 : a.seg_end[s - 1];
  const int nr = min(RPW, a.seg_end[s] - row0);
  const WT* Wp = reinterpret_cast<const WT*>(a.W[s]) + (size_t)(row0 - sbeg) * K;
  const WT* W2p = nullptr;
  if constexpr (EPI == kEpiSwiglu) W2p = reinterpret_cast<const WT*>(a.W2) + (size_t)row0 * K;

  float acc[RPW][MR], acc2[RPW][MR];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = acc2[r][m] = 0.f;

#pragma unroll 2
  for (int k = lane * VEC; k < K; k += 64 * VEC) {
    uint4 w[RPW], w2[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      w[r] = r < nr ? ld16(Wp + (size_t)r * K + k) : make_uint4(0, 0, 0, 0);
      if constexpr (EPI == kEpiSwiglu)
        w2[r] = r < nr ? ld16(W2p + (size_t)r * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float xv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const float4 t = *reinterpret_cast<const float4*>(xs + m * K + k + e);
        xv[e] = t.x;
        xv[e + 1] = t.y;
        xv[e + 2] = t.z;
        xv[e + 3] = t.w;
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float wf[VEC];
        Vec16<WT>::unpack(w[r], wf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][m] = fmaf(wf[e], xv[e], acc[r][m]);
        if constexpr (EPI == kEpiSwiglu) {
          Vec16<WT>::unpack(w2[r], wf);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc2[r][m] = fmaf(wf[e], xv[e], acc2[r][m]);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      acc[r][m] = wave_sum(acc[r][m]);
      if constexpr (EPI == kEpiSwiglu) acc2[r][m] = wave_sum(acc2[r][m]);
    }

  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (r >= nr) break;
      const int row = row0 + r;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float* o = a.out + (size_t)m * a.ldo + row;
        const float v = acc[r][m];
        if constexpr (EPI == kEpiStore) {
          *o = a.bias[s] ? v + a.bias[s][row - sbeg] : v;
        } else if constexpr (EPI == kEpiResidual) {
          *o = *o + v;
        } else {
          *o = v / (1.0f + expf(-v)) * acc2[r][m];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ QK norm + RoPE + append
// One block (D threads) per (row, head) of q, k and v.  q and k heads get
// the optional per-head RMSNorm over D and rotate-half RoPE at the row's
// position; q goes to q_out, k and v are stored into the cache row.
template <typename KT>
__global__ __launch_bounds__(128) void k_rope_append(RopeArgs a) {
  __shared__ float buf[128];
  __shared__ float red[2];
  const int hh = blockIdx.x, m = blockIdx.y, t = threadIdx.x;
  const int D = a.D, half = D >> 1;
  int slot, pos;
  row_of(a.rows, a.st, m, slot, pos);
  const int ld = (a.Hq + 2 * a.Hkv) * D;
  int kind, hd;
  if (hh < a.Hq) {
    kind = 0;
    hd = hh;
  } else if (hh < a.Hq + a.Hkv) {
    kind = 1;
    hd = hh - a.Hq;
  } else {
    kind = 2;
    hd = hh - a.Hq - a.Hkv;
  }
  const int col = (kind == 0 ? 0 : (kind == 1 ? a.Hq * D : (a.Hq + a.Hkv) * D)) + hd * D;
  float v = a.qkv[(size_t)m * ld + col + t];
  if (kind < 2 && a.qk_norm) {
    float s2 = wave_sum(v * v);
    if ((t & 63) == 0) red[t >> 6] = s2;
    __syncthreads();
    const float tot = red[0] + (D > 64 ? red[1] : 0.f);
    const float inv = 1.0f / sqrtf(tot / (float)D + a.eps);
    v = v * inv * (kind == 0 ? a.q_norm[t] : a.k_norm[t]);
  }
  if (kind < 2) {
    buf[t] = v;
    __syncthreads();
    const int i = t < half ? t : t - half;
    const float c = a.cos_t[(size_t)pos * half + i];
    const float sn = a.sin_t[(size_t)pos * half + i];
    const float x0 = buf[i], x1 = buf[i + half];
    v = t < half ? x0 * c - x1 * sn : x1 * c + x0 * sn;
  }
  if (kind == 0) {
    a.q_out[((size_t)m * a.Hq + hd) * D + t] = v;
  } else {
    void* const* kv = a.st.kv + ((size_t)slot * a.st.L + a.layer) * 2;
    const int cap = a.st.cap[slot];
    KT* dst = reinterpret_cast<KT*>(kv[kind - 1]) + ((size_t)hd * cap + pos) * D + t;
    if constexpr (sizeof(KT) == 2)
      *dst = f32_to_bf16(v);
    else
      *dst = v;
  }
}

// ------------------------------------------------------------------ attention
// Split-K decode attention.  Block (split, kv head g, row m) covers keys
// [split*chunk, min(len, (split+1)*chunk)) for the R query heads that share
// KV head g.  A key row of D elements is read by LPK lanes with 16-byte
// loads; a wave covers KPW keys per load.  Each lane group keeps an online
// softmax state (max, sum, weighted V) that is merged across groups, waves
// and (in k_attn_combine) splits, always in the same order.
template <typename KT, int D, int R>
__global__ __launch_bounds__(256) void k_attn_split(AttnArgs a) {
  constexpr int VEC = Vec16<KT>::N;
  constexpr int LPK = D / VEC;
  constexpr int KPW = 64 / LPK;
  constexpr int U = 2;
  __shared__ float sm[4][R], sl[4][R];
  __shared__ float sacc[4][R][D];

  const int split = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  int slot, pos;
  row_of(a.rows, a.st, m, slot, pos);
  const int len = pos + 1;
  const int k0 = split * a.chunk;
  if (k0 >= len) return;
  const int k1 = min(len, k0 + a.chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPK, dl = (lane % LPK) * VEC;
  const int cap = a.st.cap[slot];
  void* const* kvp = a.st.kv + ((size_t)slot * a.st.L + a.layer) * 2;
  const KT* Kb = reinterpret_cast<const KT*>(kvp[0]) + (size_t)g * cap * D + dl;
  const KT* Vb = reinterpret_cast<const KT*>(kvp[1]) + (size_t)g * cap * D + dl;

  float qv[R][VEC];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float* qp = a.q + ((size_t)m * a.Hq + g * R + j) * D + dl;
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[j][e] = qp[e] * a.scale;
  }
  float mx[R], ls[R], acc[R][VEC];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    mx[j] = -1e30f;
    ls[j] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[j][e] = 0.f;
  }

  for (int kb = k0 + wave * KPW * U; kb < k1; kb += 4 * KPW * U) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = kb + u * KPW + sub;
      ok[u] = key < k1;
      kr[u] = ok[u] ? ld16(Kb + (size_t)key * D) : make_uint4(0, 0, 0, 0);
      vr[u] = ok[u] ? ld16(Vb + (size_t)key * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC], vf[VEC];
      Vec16<KT>::unpack(kr[u], kf);
      Vec16<KT>::unpack(vr[u], vf);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) s = fmaf(qv[j][e], kf[e], s);
#pragma unroll
        for (int off = LPK >> 1; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
        if (ok[u]) {
          const float nm = fmaxf(mx[j], s);
          const float c = expf(mx[j] - nm);
          const float p = expf(s - nm);
          ls[j] = ls[j] * c + p;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(acc[j][e], c, p * vf[e]);
          mx[j] = nm;
        }
      }
    }
  }

  // merge the KPW key groups of the wave (lanes with equal dl)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float om = __shfl_xor(mx[j], off, 64);
      const float ol = __shfl_xor(ls[j], off, 64);
      const float nm = fmaxf(mx[j], om);
      const float ca = expf(mx[j] - nm), cb = expf(om - nm);
      ls[j] = ls[j] * ca + ol * cb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float oa = __shfl_xor(acc[j][e], off, 64);
        acc[j][e] = acc[j][e] * ca + oa * cb;
      }
      mx[j] = nm;
    }
  }
  if (lane < LPK) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (lane == 0) {
        sm[wave][j] = mx[j];
        sl[wave][j] = ls[j];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) sacc[wave][j][dl + e] = acc[j][e];
    }
  }
  __syncthreads();
  // merge the 4 waves in order and write this split's partial state
  for (int idx = tid; idx < R * D; idx += 256) {
    const int j = idx / D, d = idx % D;
    float M = sm[0][j];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm[w][j]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float c = expf(sm[w][j] - M);
      l += sl[w][j] * c;
      o += sacc[w][j][d] * c;
    }
    const size_t base = ((size_t)m * a.Hq + g * R + j) * a.nsplit_max + split;
    a.pacc[base * D + d] = o;
    if (d == 0) {
      a.pml[base * 2] = M;
      a.pml[base * 2 + 1] = l;
    }
  }
}

// o[m, h*D + d] = sum_s acc_s[d] e^(m_s - M) / sum_s l_s e^(m_s - M)
template <int D>
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  const int h = blockIdx.x, m = blockIdx.y, t = threadIdx.x;
  int slot, pos;
  row_of(a.rows, a.st, m, slot, pos);
  const int ns = (pos + 1 + a.chunk - 1) / a.chunk;
  const size_t base = ((size_t)m * a.Hq + h) * a.nsplit_max;
  float M = -1e30f;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.pml[(base + s) * 2]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float c = expf(a.pml[(base + s) * 2] - M);
    l += a.pml[(base + s) * 2 + 1] * c;
    o += a.pacc[(base + s) * D + t] * c;
  }
  a.o[((size_t)m * a.Hq + h) * D + t] = o / l;
}

// ------------------------------------------------------------------ slot bookkeeping
__global__ void k_advance(SlotTables st, RowMap rows, int M) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (rows.mode == kRowsPrefill) {
    if (m == 0) st.pos[rows.slot0] = M;
  } else if (m < M) {
    st.pos[rows.slot0 + m] += 1;
  }
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
  Top2 t{-INFINITY, -INFINITY, 0x7fffffff};
  for (int i = lo + tid; i < hi; i += 256) {
    float v = z[i];
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
    a.tok[b] = t.i1;
    if (a.margin) a.margin[b] = t.v1 - t.v2;
    if (a.seen) a.seen[(size_t)b * a.nwords + (t.i1 >> 5)] |= 1u << (t.i1 & 31);
  }
}

// ------------------------------------------------------------------ generation bookkeeping
__global__ void k_record_token(const int32_t* tok, int32_t* out, int32_t* counter) {
  if (threadIdx.x == 0) {
    const int k = *counter;
    out[k] = *tok;
    *counter = k + 1;
  }
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

template <typename WT, int MR, int EPI, bool NORM>
static void gemv_dispatch_rpw(const GemvArgs& a, hipStream_t s) {
  // rows per wave: as many as keep >= 512 workgroups in flight
  const int n = a.N;
  const size_t lds = (size_t)MR * a.K * sizeof(float);
  if ((n + 15) / 16 >= 512) {
    hipLaunchKernelGGL((k_gemv<WT, MR, 4, EPI, NORM>), dim3((n + 15) / 16), dim3(256), lds, s, a);
  } else if ((n + 7) / 8 >= 512) {
    hipLaunchKernelGGL((k_gemv<WT, MR, 2, EPI, NORM>), dim3((n + 7) / 8), dim3(256), lds, s, a);
  } else {
    hipLaunchKernelGGL((k_gemv<WT, MR, 1, EPI, NORM>), dim3((n + 3) / 4), dim3(256), lds, s, a);
  }
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
      gemv_dispatch_rpw<WT, 2, EPI, NORM>(b, s);
    else
      gemv_dispatch_rpw<WT, 1, EPI, NORM>(b, s);
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

hipError_t launch_gemv(const GemvArgs& a, int epi, bool norm, int bf16, hipStream_t s) {
  if (bf16)
    gemv_dispatch<uint16_t>(a, epi, norm, s);
  else
    gemv_dispatch<float>(a, epi, norm, s);
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeArgs& a, int bf16, hipStream_t s) {
  dim3 grid(a.Hq + 2 * a.Hkv, a.M);
  if (bf16)
    hipLaunchKernelGGL(k_rope_append<uint16_t>, grid, dim3(a.D), 0, s, a);
  else
    hipLaunchKernelGGL(k_rope_append<float>, grid, dim3(a.D), 0, s, a);
  return hipGetLastError();
}

template <typename KT, int D>
static void attn_dispatch_r(const AttnArgs& a, int r, dim3 grid, hipStream_t s) {
  switch (r) {
    case 1: hipLaunchKernelGGL((k_attn_split<KT, D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn_split<KT, D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn_split<KT, D, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_attn_split<KT, D, 8>), grid, dim3(256), 0, s, a); break;
  }
}

hipError_t launch_attention(const AttnArgs& a, int bf16, int D, int r, hipStream_t s) {
  dim3 grid(a.nsplit_max, a.Hkv, a.M);
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
  dim3 cgrid(a.Hq, a.M);
  if (D == 64)
    hipLaunchKernelGGL(k_attn_combine<64>, cgrid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_combine<128>, cgrid, dim3(128), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_advance(const SlotTables& st, RowMap rows, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_advance, dim3((M + 255) / 256), dim3(256), 0, s, st, rows, M);
  return hipGetLastError();
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
  hipLaunchKernelGGL(k_argmax_final, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_record_token(const int32_t* tok, int32_t* out, int32_t* counter,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_record_token, dim3(1), dim3(64), 0, s, tok, out, counter);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace atd
