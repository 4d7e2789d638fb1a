// Linear layers: Y = X W^T with fused epilogues.
//
// Kernels sharing one epilogue interface (epilogue.hpp):
//  * gemm_tile    bf16 MFMA, 128 features x 128 tokens per workgroup, K staged
//                 through LDS in 64-wide double-buffered slices (prefill).
//  * gemm_f32     float32 FMA (the fp32 model), one output pair per thread.
// Up to 64 token rows go to the weight-streaming GEMV kernel (gemv.hip).
//
// MFMA orientation: weights are the A operand (rows = output features) and
// tokens the B operand, so a lane's four accumulators of a 16x16 tile are four
// consecutive features of one token -- the adjacent feature pairs the QKV
// (rotate-half) and SwiGLU epilogues need are in the same lane.
#include "epilogue.hpp"

namespace q2 {

namespace {

constexpr int TB_N = 128;   // features per workgroup (tile kernel)
constexpr int TB_M = 128;   // tokens per workgroup
constexpr int TB_K = 64;    // K slice per LDS stage
constexpr int LDS_STRIDE = TB_K + 8;  // bf16 elements per LDS row (+16 B padding: conflict-free b128 reads)

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ------------------------------------------------------------------ tile kernel

template <typename T, int EK>
__global__ __launch_bounds__(256) void gemm_tile_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                        const uint16_t* __restrict__ X, int64_t ldx, int N,
                                                        int M, int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][TB_N * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][TB_M * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int f0 = blockIdx.y * TB_N;
  const int m0 = blockIdx.x * TB_M;
  const int wf = (wave >> 1) * 64;  // wave's feature offset in the tile
  const int wt = (wave & 1) * 64;   // wave's token offset in the tile

  // global -> register staging: each thread moves 4 rows x 16 B of W and of X per slice
  const int lrow = tid >> 3;        // 0..31
  const int lchunk = (tid & 7) * 8; // element offset inside the 64-wide slice
  uint4 rw[4], rx[4];

  auto load_slice = [&](int k0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = lrow + 32 * s;
      const int k = k0 + lchunk;
      uint4 z = {0, 0, 0, 0};
      rw[s] = (f0 + r < N && k < K) ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(f0 + r) * ldw + k) : z;
      rx[s] = (m0 + r < M && k < K) ? *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(m0 + r) * ldx + k) : z;
    }
  };
  auto store_slice = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = lrow + 32 * s;
      *reinterpret_cast<uint4*>(&sW[buf][r * LDS_STRIDE + lchunk]) = rw[s];
      *reinterpret_cast<uint4*>(&sX[buf][r * LDS_STRIDE + lchunk]) = rx[s];
    }
  };

  floatx4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + TB_K - 1) / TB_K;
  load_slice(0);
  store_slice(0);
  __syncthreads();

  const int frow = lane & 15;
  const int fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slice((kt + 1) * TB_K);
#pragma unroll
    for (int kk = 0; kk < TB_K; kk += 32) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&sW[buf][(wf + i * 16 + frow) * LDS_STRIDE + kk + fk]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&sX[buf][(wt + j * 16 + frow) * LDS_STRIDE + kk + fk]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slice(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds features 4*(lane/16)+r of token lane%16 in each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = f0 + wf + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wt + j * 16 + (lane & 15);
      if (m >= M) continue;
      if (f < N) epi_pair<T, EK>(epi, m, f, acc[i][j][0], acc[i][j][1], f + 1 < N);
      if (f + 2 < N) epi_pair<T, EK>(epi, m, f + 2, acc[i][j][2], acc[i][j][3], f + 3 < N);
    }
  }
}

// ------------------------------------------------------------------ float32 kernel

template <int EK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ W, int64_t ldw,
                                                       const float* __restrict__ X, int64_t ldx, int N, int M,
                                                       int K, Epi epi) {
  const int npairs = (N + 1) >> 1;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(npairs) * M) return;
  const int m = static_cast<int>(idx / npairs);
  const int n = static_cast<int>(idx - static_cast<int64_t>(m) * npairs) * 2;
  const bool has1 = n + 1 < N;
  const float* x = X + static_cast<int64_t>(m) * ldx;
  const float* w0 = W + static_cast<int64_t>(n) * ldw;
  const float* w1 = W + static_cast<int64_t>(has1 ? n + 1 : n) * ldw;
  float v0 = 0.f, v1 = 0.f;
  for (int k = 0; k < K; ++k) {
    const float xv = x[k];
    v0 = fmaf(xv, w0[k], v0);
    v1 = fmaf(xv, w1[k], v1);
  }
  if (EK == EPI_ARGMAX) {
    if (epi.out) {
      float* o = static_cast<float*>(epi.out) + static_cast<int64_t>(m) * epi.ldo + n;
      o[0] = v0;
      if (has1) o[1] = v1;
    }
    unsigned long long key = argmax_key(v0, n);
    if (has1) {
      unsigned long long k1 = argmax_key(v1, n + 1);
      key = k1 > key ? k1 : key;
    }
    atomicMax(epi.keys + m * KEY_ROW + ((n >> 1) % KEY_SLOTS) * KEY_STRIDE, key);
    return;
  }
  epi_pair<float, EK>(epi, m, n, v0, v1, has1);
}

template <int EK>
q2_status gemm_bf16_ek(const GemmArgs& a, hipStream_t s) {
  if constexpr (EK == EPI_ARGMAX) {
    return fail(Q2_ESHAPE, "argmax epilogue supports at most 64 rows");
  } else {
    dim3 grid(cdiv(a.M, TB_M), cdiv(a.N, TB_N));
    hipLaunchKernelGGL((gemm_tile_kernel<uint16_t, EK>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(a.W),
                       a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M, a.K, a.epi);
    return check_launch("gemm_tile");
  }
}

template <int EK>
q2_status gemm_f32_ek(const GemmArgs& a, hipStream_t s) {
  const int64_t work = static_cast<int64_t>((a.N + 1) / 2) * a.M;
  hipLaunchKernelGGL(gemm_f32_kernel<EK>, dim3(cdiv(work, 256)), dim3(256), 0, s, static_cast<const float*>(a.W),
                     a.ldw, static_cast<const float*>(a.X), a.ldx, a.N, a.M, a.K, a.epi);
  return check_launch("gemm_f32");
}

}  // namespace

q2_status gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return Q2_OK;
  Q2_CHECK(a.K % 8 == 0, Q2_ESHAPE, "bf16 linear: K=%d must be a multiple of 8", a.K);
  if (a.M <= GEMV_MAX_M) return gemv_bf16(a, s);
  Q2_CHECK(a.norm_w == nullptr, Q2_EINVAL, "fused RMSNorm needs M <= %d", GEMV_NORM_MAX_M);
  switch (a.epi.kind) {
    case EPI_STORE: return gemm_bf16_ek<EPI_STORE>(a, s);
    case EPI_RESID: return gemm_bf16_ek<EPI_RESID>(a, s);
    case EPI_SWIGLU: return gemm_bf16_ek<EPI_SWIGLU>(a, s);
    case EPI_QKV: return gemm_bf16_ek<EPI_QKV>(a, s);
    case EPI_ARGMAX: return gemm_bf16_ek<EPI_ARGMAX>(a, s);
  }
  return fail(Q2_EINVAL, "unknown epilogue %d", a.epi.kind);
}

q2_status gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return Q2_OK;
  switch (a.epi.kind) {
    case EPI_STORE: return gemm_f32_ek<EPI_STORE>(a, s);
    case EPI_RESID: return gemm_f32_ek<EPI_RESID>(a, s);
    case EPI_SWIGLU: return gemm_f32_ek<EPI_SWIGLU>(a, s);
    case EPI_QKV: return gemm_f32_ek<EPI_QKV>(a, s);
    case EPI_ARGMAX: return gemm_f32_ek<EPI_ARGMAX>(a, s);
  }
  return fail(Q2_EINVAL, "unknown epilogue %d", a.epi.kind);
}

}  // namespace q2
