// Pre-packed MXFP4 decode weights and the GEMV that streams them.
//
// Weight pre-processing as a separate load-time step, re-ordering the weights for
// the matrix instruction, is the W4A8 practice described in the Hopper CUTLASS/CuTe
// DSL post (section "The W4A8 kernel: the same four definitions, with the operands
// swapped": the weights are re-encoded and re-ordered when they are loaded, and the
// scales re-packed).  Here the same idea serves the MXFP4 decode GEMV on gfx950:
// the pre-packed layout is the register layout of the B operand of
// v_mfma_scale_f32_16x16x128_f8f6f4, so a wave's weight load is one fully
// coalesced 1 KB global_load_dwordx4 per MFMA, straight into registers (no LDS
// round trip, no swizzle), and a lane's four scale bytes for four consecutive K
// steps are one dword.
//
// Layout (G = ceil(N/16) row groups of 16 weight rows, KT = K/128 steps,
// KC = ceil(KT/4) scale chunks; lane l = 16*slot + r):
//   Bp[g][s][l][0..15] = B[16g + r][64s + 16*slot .. 64s + 16*slot + 15]
//                        (the 32 E2M1 codes of K elements 128s + 32*slot .. +31)
//   Sp[g][c][l]        = dword whose byte i is sfB[16g + r][4(4c+i) + slot]
//                        (the E8M0 scale of those 32 elements at step 4c+i)
// Rows past N hold zero codes and scale 127; steps past KT in the last chunk hold
// scale 127.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int PW = 8;          // waves per workgroup; they split K
constexpr int CH = 4;          // K steps per wave per pass (all loads of a pass in flight)

__global__ void __launch_bounds__(256)
prepack_weights_kernel(int64_t units, int N, int KT, int64_t ld, const uint8_t* __restrict__ B,
                       uint8_t* __restrict__ Bp) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int l = (int)(u & 63);
    const int64_t gs = u >> 6;
    const int s = (int)(gs % KT);
    const int64_t g = gs / KT;
    const int64_t row = 16 * g + (l & 15);
    v4i v = v4i{0, 0, 0, 0};
    if (row < N) v = *reinterpret_cast<const v4i*>(B + row * ld + (int64_t)s * 64 + (l >> 4) * 16);
    *reinterpret_cast<v4i*>(Bp + u * 16) = v;
  }
}

__global__ void __launch_bounds__(256)
prepack_scales_kernel(int64_t units, int N, int KT, int KC, int64_t lsc, const uint8_t* __restrict__ sfB,
                      uint32_t* __restrict__ Sp) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int l = (int)(u & 63);
    const int64_t gc = u >> 6;
    const int c = (int)(gc % KC);
    const int64_t g = gc / KC;
    const int64_t row = 16 * g + (l & 15);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * c + i;
      const uint32_t b = (row < N && s < KT) ? sfB[row * lsc + 4 * s + (l >> 4)] : 127u;
      w |= b << (8 * i);
    }
    Sp[u] = w;
  }
}

// One workgroup per RGW row groups; wave w takes the scale chunks
// [w*KC/PW, (w+1)*KC/PW) (whole 4-step chunks, so its scale dwords are its own) and
// walks them CH steps at a time: every weight, token and scale load of a pass is
// issued before the first wait.  The PW partial 16 x 16 tiles are then summed
// through LDS in wave order.
template <int RGW, bool BF16>
__global__ void __launch_bounds__(PW * 64)
fp4_gemv_prepacked_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                          const uint8_t* __restrict__ Bp, const uint32_t* __restrict__ Sp, void* __restrict__ D) {
  __shared__ __attribute__((aligned(16))) float red[PW][RGW][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int KT = K / 128, KC = (KT + 3) / 4;
  const int G = (N + 15) / 16;
  const int64_t ld = K / 2, lsc = K / 32;
  const int c0 = (int)((int64_t)wave * KC / PW), c1 = (int)((int64_t)(wave + 1) * KC / PW);
  const int kend = min(4 * c1, KT);            // this wave's steps: 4*c0 .. kend-1

  const uint8_t* wrow[RGW];
  const uint32_t* srow[RGW];
#pragma unroll
  for (int g = 0; g < RGW; ++g) {
    const int64_t gg = min((int64_t)blockIdx.x * RGW + g, (int64_t)G - 1);
    wrow[g] = Bp + gg * KT * 1024 + lane * 16;
    srow[g] = Sp + gg * KC * 64 + lane;
  }
  const bool tok = r < M;
  const int64_t trow = tok ? r : 0;
  // Token scale words of 4 consecutive steps are one 16-byte load when rows of scales
  // are 16-byte multiples and the base is 16-byte aligned.
  const bool vec_ts = (K & 511) == 0 && (reinterpret_cast<uintptr_t>(sfA) & 15) == 0;

  v4f acc[RGW];
#pragma unroll
  for (int g = 0; g < RGW; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int cs = c0; cs < c1; cs += CH / 4) {
    const int k0 = 4 * cs;
    v4i w[RGW][CH], t[CH];
    uint32_t ws[RGW][CH / 4];
    int ts[CH];
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      const int ks = min(k0 + s, KT - 1);
#pragma unroll
      for (int g = 0; g < RGW; ++g)
        w[g][s] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow[g] + (int64_t)ks * 1024));
    }
#pragma unroll
    for (int q = 0; q < CH / 4; ++q)
#pragma unroll
      for (int g = 0; g < RGW; ++g) ws[g][q] = srow[g][min(cs + q, KC - 1) * 64];
    if (M <= 8) {
      // Lanes r >= 8 fetch the next step of token r-8; a row rotation by 8 (DPP
      // row_ror:8) then moves it into lanes 0..7.
      const int64_t prow = min(r & 7, M - 1);
#pragma unroll
      for (int s = 0; s < CH; s += 2) {
        const int ks = min(k0 + s + (r >> 3), KT - 1);
        t[s] = *reinterpret_cast<const v4i*>(A + prow * ld + (int64_t)ks * 64 + slot * 16);
      }
    } else {
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        const int ks = min(k0 + s, KT - 1);
        t[s] = *reinterpret_cast<const v4i*>(A + trow * ld + (int64_t)ks * 64 + slot * 16);
      }
    }
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) {
      const int ks = k0 + 4 * q;
      if (vec_ts && ks + 4 <= KT) {
        const v4i w4 = *reinterpret_cast<const v4i*>(sfA + trow * lsc + ks * 4);
        ts[4 * q] = w4[0]; ts[4 * q + 1] = w4[1]; ts[4 * q + 2] = w4[2]; ts[4 * q + 3] = w4[3];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) ts[4 * q + u] = *reinterpret_cast<const int*>(sfA + trow * lsc + min(ks + u, KT - 1) * 4);
      }
    }
    if (M <= 8) {
#pragma unroll
      for (int s = 0; s < CH; s += 2)
#pragma unroll
        for (int e = 0; e < 4; ++e) t[s + 1][e] = __builtin_amdgcn_mov_dpp(t[s][e], 0x128, 0xF, 0xF, false);
    }
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      const bool ok = k0 + s < kend;
      const bool tk = ok && tok;
      const int tsc = tk ? (ts[s] >> (8 * slot)) & 255 : 127;
      const v4i tv = tk ? t[s] : v4i{0, 0, 0, 0};
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        const int wsc = ok ? (int)((ws[g][s >> 2] >> (8 * (s & 3))) & 255u) : 127;
        acc[g] = mfma_fp4_16x16<0>(w[g][s], tv, acc[g], wsc, tsc);
      }
    }
  }

  // ---- sum the PW partial tiles in wave order, store D[m][n] ----
#pragma unroll
  for (int g = 0; g < RGW; ++g) *reinterpret_cast<v4f*>(&red[wave][g][lane][0]) = acc[g];
  __syncthreads();
  if (threadIdx.x < RGW * 64) {
    const int g = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int m = l & 15;
    v4f v = *reinterpret_cast<const v4f*>(&red[0][g][l][0]);
#pragma unroll
    for (int w2 = 1; w2 < PW; ++w2) v += *reinterpret_cast<const v4f*>(&red[w2][g][l][0]);
    const int64_t n = ((int64_t)blockIdx.x * RGW + g) * 16 + 4 * (l >> 4);
    if (m < M && n < N) {
      const int avail = (int)min((int64_t)4, (int64_t)N - n);
      store_out4<BF16>(D, (int64_t)m * N + n, avail, v[0], v[1], v[2], v[3]);
    }
  }
}

template <int RGW>
hipError_t launch_rgw(const FP4Args& a, const uint32_t* Sp, hipStream_t s) {
  const int64_t G = ceil_div(a.N, 16);
  const int64_t wgs = ceil_div(G, RGW);
  if (wgs > INT32_MAX) return hipErrorInvalidConfiguration;
  if (a.bf16_out)
    hipLaunchKernelGGL((fp4_gemv_prepacked_kernel<RGW, true>), dim3((unsigned)wgs), dim3(PW * 64), 0, s, (int)a.M,
                       (int)a.N, (int)a.K, a.A, a.sfA, a.B, Sp, a.D);
  else
    hipLaunchKernelGGL((fp4_gemv_prepacked_kernel<RGW, false>), dim3((unsigned)wgs), dim3(PW * 64), 0, s, (int)a.M,
                       (int)a.N, (int)a.K, a.A, a.sfA, a.B, Sp, a.D);
  return hipGetLastError();
}

}  // namespace

void gemv_prepack_sizes(int64_t N, int64_t K, int64_t* weight_bytes, int64_t* scale_bytes) {
  const int64_t G = ceil_div(N, 16), KT = K / 128;
  *weight_bytes = G * KT * 1024;
  *scale_bytes = G * ceil_div(KT, 4) * 256;
}

hipError_t launch_gemv_prepack(int64_t N, int64_t K, const uint8_t* B, const uint8_t* sfB, uint8_t* Bp,
                               uint32_t* Sp, hipStream_t s) {
  const int64_t G = ceil_div(N, 16), KT = K / 128, KC = ceil_div(KT, 4);
  const int64_t cap = device_cus() * 8;
  const int64_t wu = G * KT * 64, su = G * KC * 64;
  const unsigned gw = (unsigned)(ceil_div(wu, 256) < cap ? ceil_div(wu, 256) : cap);
  const unsigned gs = (unsigned)(ceil_div(su, 256) < cap ? ceil_div(su, 256) : cap);
  hipLaunchKernelGGL(prepack_weights_kernel, dim3(gw), dim3(256), 0, s, wu, (int)N, (int)KT, K / 2, B, Bp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prepack_scales_kernel, dim3(gs), dim3(256), 0, s, su, (int)N, (int)KT, (int)KC, K / 32, sfB, Sp);
  return hipGetLastError();
}

// a.B is the pre-packed weight buffer Bp; Sp the pre-packed scales.
hipError_t launch_fp4_gemv_prepacked(const FP4Args& a, const uint32_t* Sp, hipStream_t s) {
  // Two row groups per workgroup share each wave's token fragments; one when that
  // would leave fewer workgroups than CUs.
  if (ceil_div(ceil_div(a.N, 16), 2) >= device_cus()) return launch_rgw<2>(a, Sp, s);
  return launch_rgw<1>(a, Sp, s);
}

}  // namespace fp4g
