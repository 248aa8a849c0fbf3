// Latent-space decode attention: the vector-ALU kernel (fp32 debug mode and any head count) and
// the log-sum-exp merge of page ranges that split a sequence.
//
// Per sequence b and head h (DeepSeek-V2 explainer, Steps 6-8): every cached row [c_t | k^R_t]
// is scored by one 576-long dot product with the latent-form query [W_UK^T q_nope | q^R] -- the
// content score and the RoPE score add inside the softmax -- and the softmax weights average the
// notes c_t.  The running softmax is kept in base 2: s' = s * scale * log2(e).
#include <type_traits>

#include "mla_device.h"

namespace mla {

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s);

namespace {

constexpr int kTile = 32;             // tokens per LDS tile
constexpr int kRowDw = kRow / 2 + 1;  // 289 dwords per LDS row: consecutive rows start on different banks
constexpr int kHG = 8;                // heads per workgroup (32 lanes each)
constexpr int kQStride = kRow + 2;    // fp32 query rows, padded

template <typename QT, typename OT>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeParams p) {
  __shared__ float q_s[kHG][kQStride];
  __shared__ uint32_t kv_s[kTile][kRowDw];
  __shared__ float s_s[kHG][kTile + 1];

  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  const int h0 = blockIdx.y * kHG;
  const int hh = tid >> 5;     // head within the group
  const int j32 = tid & 31;    // token of the tile for its score, dword lane for the weighted sum
  const QT* q_abs = static_cast<const QT*>(p.q_abs);

  SegmentWalker walk;
  walk.init(p.seq_lens, p.batch, p.num_units, w);
  Segment seg;
  while (walk.next(seg)) {
    const int b = seg.b;
    __syncthreads();
    {
      // The heads' query rows as groups of 8 numbers (16 bytes in bf16, 32 in fp32), every load in
      // flight before the first store.
      constexpr int kGroups = kHG * kRow / 8;
      constexpr int kIters = (kGroups + 255) / 256;
      float qv[kIters][8];
#pragma unroll
      for (int u = 0; u < kIters; ++u) {
        const int i = tid + 256 * u;
        if (i < kGroups) {
          const QT* src = q_abs + ((size_t)b * p.heads + h0 + i / (kRow / 8)) * kRow + 8 * (i % (kRow / 8));
          if constexpr (sizeof(QT) == 2) {
            const uint4 v = *reinterpret_cast<const uint4*>(src);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              qv[u][2 * j] = bf16_lo(w4[j]);
              qv[u][2 * j + 1] = bf16_hi(w4[j]);
            }
          } else {
            const float4 a = *reinterpret_cast<const float4*>(src);
            const float4 c = *reinterpret_cast<const float4*>(src + 4);
            qv[u][0] = a.x; qv[u][1] = a.y; qv[u][2] = a.z; qv[u][3] = a.w;
            qv[u][4] = c.x; qv[u][5] = c.y; qv[u][6] = c.z; qv[u][7] = c.w;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kIters; ++u) {
        const int i = tid + 256 * u;
        if (i < kGroups) {
#pragma unroll
          for (int j = 0; j < 8; ++j) q_s[i / (kRow / 8)][8 * (i % (kRow / 8)) + j] = qv[u][j];
        }
      }
    }
    float acc[16];  // latent dims 64 j + 2 j32 + {0, 1}, j < 8
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;  // the same in the 32 lanes of a head

    const int t_begin = seg.page0 * kPage;
    const int t_end = min(seg.page1 * kPage, seg.len);
    const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
    // A tile is 32 x 72 pieces of 16 bytes, nine per thread; the next tile's pieces are loaded into
    // registers while the current one is computed.  Rows past the end re-read the last valid token
    // (finite, masked below), so no slot beyond the sequence and no unused block-table entry is
    // ever touched.
    constexpr int kPieces = kTile * (kRow / 8) / 256;
    uint4 pre[kPieces];
    auto load_tile = [&](int t0) {
      const int nt = min(kTile, t_end - t0);
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        const int i = tid + 256 * u;
        const int r = i / (kRow / 8), c = i % (kRow / 8);
        const int t = t0 + min(r, nt - 1);
        const int page = bt[t / kPage];
        pre[u] = reinterpret_cast<const uint4*>(p.cache + ((size_t)page * kPage + (t % kPage)) * kRow)[c];
      }
    };
    if (t_begin < t_end) load_tile(t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
      const int nt = min(kTile, t_end - t0);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        const int i = tid + 256 * u;
        uint32_t* dst = &kv_s[i / (kRow / 8)][(i % (kRow / 8)) * 4];
        dst[0] = pre[u].x; dst[1] = pre[u].y; dst[2] = pre[u].z; dst[3] = pre[u].w;
      }
      __syncthreads();
      if (t0 + kTile < t_end) load_tile(t0 + kTile);
      float s0 = 0.f, s1 = 0.f;  // even and odd dims of the score of token j32
      {
        const uint32_t* r0 = kv_s[j32];
        const float* qh = q_s[hh];
#pragma unroll 8
        for (int k2 = 0; k2 < kRow / 2; ++k2) {
          const uint32_t a = r0[k2];
          s0 = fmaf(qh[2 * k2], bf16_lo(a), s0);
          s1 = fmaf(qh[2 * k2 + 1], bf16_hi(a), s1);
        }
        s0 = (j32 < nt) ? (s0 + s1) * p.scale_log2 : -INFINITY;
      }
      // Online softmax of the head's 32 scores across its 32 lanes; token 0 of a tile is always
      // valid, so the tile maximum is finite.
      float mx = s0;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      const float e0 = exp2f(s0 - m_new);
      float sum = e0;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 32);
      l_run = l_run * alpha + sum;
      m_run = m_new;
      s_s[hh][j32] = e0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= alpha;
      for (int t = 0; t < kTile; ++t) {
        const float pt = s_s[hh][t];
        const uint32_t* rv = kv_s[t];
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // latent dims 64 j + 2 j32 + {0, 1}
          const uint32_t v = rv[j * 32 + j32];
          acc[2 * j] = fmaf(pt, bf16_lo(v), acc[2 * j]);
          acc[2 * j + 1] = fmaf(pt, bf16_hi(v), acc[2 * j + 1]);
        }
      }
    }
    // Un-normalised partial sum plus (reference max, softmax sum); the merge kernel finishes it.
    const size_t part = ((size_t)w + b) * p.heads + h0 + hh;
    float* o = p.ws_o + part * kDc;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<float2*>(o + 64 * j + 2 * j32) = make_float2(acc[2 * j], acc[2 * j + 1]);
    if (j32 == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * part) = make_float2(m_run, l_run);
  }
}

// Eight consecutive outputs from one lane (one 16-byte store for bf16, two for fp32).
__device__ __forceinline__ void store8(uint16_t* o, size_t i, const float* x) {
  uint4 v;
  v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
  v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
  v.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
  v.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
  *reinterpret_cast<uint4*>(o + i) = v;
}
__device__ __forceinline__ void store8(float* o, size_t i, const float* x) {
  *reinterpret_cast<float4*>(o + i) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(o + i + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Finishes every sequence: combines its pieces (one per work unit it touches, stored at slot
// unit + sequence), divides by the softmax sum and writes o_lat and lse.
//   M = max_s m_s;  w_s = 2^(m_s - M);  o = sum_s w_s O_s / sum_s w_s l_s;  lse = ln2 (M + log2 sum_s w_s l_s)
// where O_s is a piece's un-normalised sum (fp32 pieces) or l_s times its normalised bf16 sum
// (bf16 pieces).  One workgroup of 256 lanes per (sequence, HPW heads): 256 / HPW lanes per head,
// HPW / 2 groups of 4 latent dims per lane.  Pieces are read a chunk at a time (256 bytes in flight
// per lane) and folded in with a running maximum (the sums are rescaled when a chunk raises it), so
// the partials are read once.  HPW trades parallelism (long sequences, few of them) against the
// fixed per-workgroup cost (many short sequences).
template <typename OT, int HPW, bool PB>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  constexpr int kTPH = 256 / HPW;      // lanes per head
  constexpr int kF4 = HPW / 2;         // groups of 4 dims per lane per piece
  constexpr int kChunk = (PB ? 32 : 16) / kF4;  // pieces per chunk: 256 bytes in flight per lane
  const int b = blockIdx.x;
  const int h = blockIdx.y * HPW + threadIdx.x / kTPH;
  const int j = threadIdx.x % kTPH;
  const int len = p.seq_lens[b];
  const int4 su_entry = seq_units_entry(p, b);
  const long long np = pages_of(len);
  OT* o = static_cast<OT*>(p.o_lat);
  const size_t ob = ((size_t)b * p.heads + h) * kDc;
  if (np == 0) {
#pragma unroll
    for (int f = 0; f < kF4; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) Elem<OT>::store(o, ob + 4 * (j + kTPH * f) + i, 0.f);
    if (p.lse && j == 0) p.lse[(size_t)b * p.heads + h] = -INFINITY;
    return;
  }
  const SeqUnits su = seq_units_of(p, b, np, su_entry);
  const int wf = su.wf, wl = su.wl;
  auto live = [&](int w) { return su.live(w); };
  auto slot = [&](int w) { return ((size_t)w + b) * p.heads + h; };

  float mx = -INFINITY;
  float4 acc[kF4];
#pragma unroll
  for (int f = 0; f < kF4; ++f) acc[f] = make_float4(0.f, 0.f, 0.f, 0.f);
  float sum = 0.f;
  for (int w0 = wf; w0 <= wl; w0 += kChunk) {
    // bf16 pieces stay packed (two registers per 4 dims) until they are used
    typedef typename std::conditional<PB, uint2, float4>::type Raw;
    Raw v[kChunk][kF4];
    float2 ml[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (w0 + u <= wl) {
        const float* src = p.ws_o + slot(w0 + u) * kDc;
#pragma unroll
        for (int f = 0; f < kF4; ++f) {
          const int d = 4 * (j + kTPH * f);
          if constexpr (PB) v[u][f] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(src) + d);
          else v[u][f] = *reinterpret_cast<const float4*>(src + d);
        }
        ml[u] = *reinterpret_cast<const float2*>(p.ws_ml + 2 * slot(w0 + u));
      }
    }
    bool use[kChunk];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      use[u] = w0 + u <= wl && live(w0 + u);
      if (use[u]) cm = fmaxf(cm, ml[u].x);
    }
    if (cm > mx) {  // exp2(-inf) = 0 covers the first chunk
      const float r = exp2f(mx - cm);
      sum *= r;
#pragma unroll
      for (int f = 0; f < kF4; ++f) {
        acc[f].x *= r; acc[f].y *= r; acc[f].z *= r; acc[f].w *= r;
      }
      mx = cm;
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (!use[u]) continue;
      const float wgt = exp2f(ml[u].x - mx);
      const float wl_s = wgt * ml[u].y;
      sum += wl_s;
      const float wo = PB ? wl_s : wgt;
#pragma unroll
      for (int f = 0; f < kF4; ++f) {
        float4 x;
        if constexpr (PB) x = make_float4(bf16_lo(v[u][f].x), bf16_hi(v[u][f].x), bf16_lo(v[u][f].y), bf16_hi(v[u][f].y));
        else x = v[u][f];
        acc[f].x = fmaf(wo, x.x, acc[f].x); acc[f].y = fmaf(wo, x.y, acc[f].y);
        acc[f].z = fmaf(wo, x.z, acc[f].z); acc[f].w = fmaf(wo, x.w, acc[f].w);
      }
    }
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int f = 0; f < kF4; ++f) {
    const size_t e = ob + 4 * (j + kTPH * f);
    Elem<OT>::store(o, e, acc[f].x * inv);
    Elem<OT>::store(o, e + 1, acc[f].y * inv);
    Elem<OT>::store(o, e + 2, acc[f].z * inv);
    Elem<OT>::store(o, e + 3, acc[f].w * inv);
  }
  if (p.lse && j == 0) p.lse[(size_t)b * p.heads + h] = (mx + log2f(sum)) * 0.69314718055994531f;
}

template <typename T>
hipError_t launch_valu(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_valu_kernel<T, T>), dim3(p.num_units, p.heads / kHG), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Merge for bf16 pieces: one workgroup per (sequence, head).  Its 256 lanes are four groups of 64;
// lane l of group g holds latent dims 8 (l % 64) .. + 7 and folds in pieces g, g + 4, ... of the
// sequence with a running maximum, all of its loads in flight together (one 16-byte load and one
// 8-byte (max, sum) load per piece); the four groups are then combined through LDS.
template <typename OT>
__global__ __launch_bounds__(256) void merge_pieces_kernel(DecodeParams p) {
  constexpr int kGroups = 4;
  constexpr int kChunk = 16;  // pieces per group in flight
  __shared__ float red_acc[kGroups][kDc];
  __shared__ float red_ms[kGroups][2];
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int g = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int len = p.seq_lens[b];
  const int4 su_entry = seq_units_entry(p, b);
  const long long np = pages_of(len);
  OT* o = static_cast<OT*>(p.o_lat);
  const size_t ob = ((size_t)b * p.heads + h) * kDc;
  if (np == 0) {
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) Elem<OT>::store(o, ob + 8 * l + i, 0.f);
      if (p.lse && l == 0) p.lse[(size_t)b * p.heads + h] = -INFINITY;
    }
    return;
  }
  const SeqUnits su = seq_units_of(p, b, np, su_entry);
  const int wf = su.wf, wl = su.wl;
  auto live = [&](int w) { return su.live(w); };
  auto slot = [&](int w) { return ((size_t)w + b) * p.heads + h; };

  float mx = -INFINITY, sum = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int w0 = wf + g; w0 <= wl; w0 += kGroups * kChunk) {
    uint4 v[kChunk];
    float2 ml[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int w = w0 + kGroups * u;
      if (w <= wl) {
        v[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.ws_o + slot(w) * kDc) + 8 * l);
        ml[u] = *reinterpret_cast<const float2*>(p.ws_ml + 2 * slot(w));
      }
    }
    bool use[kChunk];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int w = w0 + kGroups * u;
      use[u] = w <= wl && live(w);
      if (use[u]) cm = fmaxf(cm, ml[u].x);
    }
    if (cm > mx) {
      const float r = exp2f(mx - cm);
      sum *= r;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= r;
      mx = cm;
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (!use[u]) continue;
      const float wl_s = exp2f(ml[u].x - mx) * ml[u].y;
      sum += wl_s;
      const uint32_t raw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wl_s, bf16_lo(raw[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wl_s, bf16_hi(raw[i]), acc[2 * i + 1]);
      }
    }
  }
  // combine the four groups
#pragma unroll
  for (int i = 0; i < 8; ++i) red_acc[g][8 * l + i] = acc[i];
  if (l == 0) {
    red_ms[g][0] = mx;
    red_ms[g][1] = sum;
  }
  __syncthreads();
  if (g == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kGroups; ++q) M = fmaxf(M, red_ms[q][0]);
    float wq[kGroups], tot = 0.f;
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      wq[q] = exp2f(red_ms[q][0] - M);  // a group with no piece has max -inf and weight 0
      tot += wq[q] * red_ms[q][1];
    }
    const float inv = 1.f / tot;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = 0.f;
#pragma unroll
      for (int q = 0; q < kGroups; ++q) x[i] = fmaf(wq[q], red_acc[q][8 * l + i], x[i]);
      x[i] *= inv;
    }
    store8(o, ob + 8 * l, x);
    if (p.lse && l == 0) p.lse[(size_t)b * p.heads + h] = (M + log2f(tot)) * 0.69314718055994531f;
  }
}

// Heads per merge workgroup: as many as keep at least one workgroup per compute unit.
template <typename T, bool PB>
hipError_t launch_merge(const DecodeParams& p, hipStream_t s) {
  const long long rows = (long long)p.batch * p.heads;
  if (rows >= 8LL * kNumCUs && p.heads % 8 == 0)
    hipLaunchKernelGGL((merge_kernel<T, 8, PB>), dim3(p.batch, p.heads / 8), dim3(256), 0, s, p);
  else if (rows >= 4LL * kNumCUs && p.heads % 4 == 0)
    hipLaunchKernelGGL((merge_kernel<T, 4, PB>), dim3(p.batch, p.heads / 4), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((merge_kernel<T, 2, PB>), dim3(p.batch, p.heads / 2), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_pieces(DecodeParams& p, bool f32, hipStream_t s) {
  if (p.fp6 && (f32 || !mfma_supported(p))) return hipErrorNotSupported;  // matrix-core kernel only
  if (f32) {  // debug mode: fp32 everywhere, fp32 pieces
    p.partial_bf16 = 0;
    p.seq_units = nullptr;
    return launch_valu<float>(p, s);
  }
  if (mfma_supported(p)) {  // the matrix-core kernel writes normalised bf16 pieces
    p.partial_bf16 = 1;
    return launch_decode_mfma(p, s);
  }
  p.partial_bf16 = 0;
  p.seq_units = nullptr;
  return launch_valu<uint16_t>(p, s);
}

hipError_t launch_decode(const DecodeParams& params, bool f32, hipStream_t s) {
  DecodeParams p = params;
  hipError_t e = launch_decode_pieces(p, f32, s);
  if (e != hipSuccess) return e;
  if (f32) return launch_merge<float, false>(p, s);
  if (!p.partial_bf16) return launch_merge<uint16_t, false>(p, s);
  if (p.num_units >= 16 * p.batch) {  // long sequences: many pieces each
    hipLaunchKernelGGL(merge_pieces_kernel<uint16_t>, dim3(p.batch, p.heads), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  return launch_merge<uint16_t, true>(p, s);
}

}  // namespace mla
