// Fast fp32 WBMM forward for w = 7 on NCHW 56x56 images (64 windows per image), table input.
// With d = 49 a window needs 2 x 49 flops per output pixel against 8 bytes of map traffic, so
// the kernel streams the map through HBM with the matrix cores beside it [gecl.asia reading
// notes, "Core Idea": one per-channel matrix from the relative-position table, shared by every
// window].
//
// Persistent waves, no LDS and no barriers: each wave walks a run of (channel, image) planes,
// a plane at a time as 4 wave-units of 16 windows (two window rows of 8), on
// v_mfma_f32_16x16x4f32 (16 pixel slots x 16 windows x 4 K per instruction):
//   * pixel slots and K are window rows padded to 8 (slot = row * 8 + column, column 7 empty),
//     so the 49 outputs take 4 row tiles (64 slots) and the 49 inputs 14 K steps (56 slots);
//   * the table operand M[slot][k] is the same for every window of a channel: 4 tiles x 14 steps
//     = 56 registers per lane, formed from the table when the channel changes (zero for padding
//     slots), so the steady state reads no table at all;
//   * the window operand goes from HBM straight into registers: lane (window n, K group g) needs
//     columns g and g + 4 of each of its window's 7 rows (column 7 is padding), 14 loads per
//     wave-unit, issued three wave-units ahead;
//   * a lane's four accumulators of a tile are 4 consecutive slots of one window row: columns
//     0..3 leave as one 16-byte store, columns 4..6 as an 8-byte and a 4-byte store.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

#include <atomic>

namespace wbmm {
namespace {

constexpr int F7_WS = 7, F7_IW = 56, F7_PLANE = F7_IW * F7_IW;
constexpr int F7_L1 = 2 * F7_WS - 1, F7_L = F7_L1 * F7_L1;  // 13, 169
constexpr int F7_NT = 4;     // row tiles of 16 slots
constexpr int F7_KS = 14;    // K steps of 4
constexpr int F7_WPI = 4;    // wave-units per image
constexpr int F7_PF = 3;     // wave-units in flight ahead of the one contracted

struct F7Args {
  int B, C;
  long long items;  // C * B planes, channel-major (item = c * B + b)
  const float* x;
  const float* T;
  float* y;
  float* z;         // a second copy of the output, or null
};

typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f2u __attribute__((ext_vector_type(2), aligned(4)));

__global__ void __launch_bounds__(256) k_fwd_f32_w7(F7Args a) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const long long nw = (long long)gridDim.x * 4;
  const long long gw = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long i0 = gw * a.items / nw, i1 = (gw + 1) * a.items / nw;
  if (i0 >= i1) return;  // uniform over the wave

  // wave-unit q of the stream: plane i0 + q / 4, unit q % 4 (window rows 2u, 2u + 1)
  const long long nq = (i1 - i0) * F7_WPI;
  // this lane's window within a unit: window row 2u + n / 8, window column n % 8
  const int wrow = n >> 3, wcol = n & 7;
  auto plane_off = [&](long long q) {
    const long long it = i0 + q / F7_WPI;
    const int c = (int)(it / a.B), b = (int)(it - (long long)c * a.B);
    return ((size_t)b * a.C + c) * F7_PLANE;
  };
  // element offset of (window row 0 of the unit, column g) of this lane's window
  auto unit_off = [&](long long q) {
    const int u = (int)(q % F7_WPI);
    return plane_off(q) + (size_t)((2 * u + wrow) * F7_WS) * F7_IW + wcol * F7_WS + g;
  };
  // step s: row s / 2, column g + 4 (s % 2); column 7 (g = 3, odd s) is padding
  auto issue = [&](long long q, float (&v)[F7_KS]) {
    const float* src = a.x + unit_off(q < nq ? q : nq - 1);
#pragma unroll
    for (int s = 0; s < F7_KS; ++s) {
      const int off = (s >> 1) * F7_IW + ((s & 1) ? 4 : 0);
      // the padding column reads column 3 of the row and is zeroed (no load leaves the window)
      const float t = src[(g == 3 && (s & 1)) ? (s >> 1) * F7_IW : off];
      v[s] = (g == 3 && (s & 1)) ? 0.f : t;
    }
  };

  float am[F7_NT][F7_KS];
  int table_c = -1;
  auto form_table = [&](int c) {
    const float* Tc = a.T + (size_t)c * F7_L;
#pragma unroll
    for (int t = 0; t < F7_NT; ++t)
#pragma unroll
      for (int s = 0; s < F7_KS; ++s) {
        const int m = 16 * t + n, k = 4 * s + g;
        const int py = m >> 3, px = m & 7, qy = k >> 3, qx = k & 7;
        const bool ok = py < F7_WS && px < F7_WS && qx < F7_WS;
        const float v = Tc[ok ? (py - qy + F7_WS - 1) * F7_L1 + (px - qx + F7_WS - 1) : 0];
        am[t][s] = ok ? v : 0.f;
      }
  };

  static_assert(F7_PF + 1 == F7_WPI, "one ring turn per plane");
  float ring[F7_WPI][F7_KS];
#pragma unroll
  for (int p = 0; p < F7_PF; ++p) issue(p, ring[p]);
  // a plane (4 wave-units) per iteration, unit h in ring slot h; the wave-unit F7_PF ahead goes
  // into the slot the previous unit has left
  for (long long q0 = 0; q0 < nq; q0 += F7_WPI) {
#pragma unroll
    for (int h = 0; h < F7_WPI; ++h) {
      const long long q = q0 + h;
      issue(q + F7_PF, ring[(h + F7_PF) % F7_WPI]);
      const long long it = i0 + q / F7_WPI;
      const int c = (int)(it / a.B);
      if (c != table_c) {  // uniform
        form_table(c);
        table_c = c;
      }
      v4f acc[F7_NT];
#pragma unroll
      for (int t = 0; t < F7_NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < F7_KS; ++s)
#pragma unroll
        for (int t = 0; t < F7_NT; ++t) acc[t] = mfma_f32(am[t][s], ring[h][s], acc[t]);
      // lane (window n, g) holds slots 16t + 4g + r = row 2t + g / 2, columns 4 (g % 2) + r
      const size_t wo = unit_off(q) - g;  // this lane's window origin
#pragma unroll
      for (int t = 0; t < F7_NT; ++t) {
        const int py = 2 * t + (g >> 1);
        if (py >= F7_WS) continue;  // t = 3, g >= 2: padding row
        const size_t o = wo + (size_t)py * F7_IW + 4 * (g & 1);
        const v4f d = acc[t];
        if ((g & 1) == 0) {
          *(f4u*)(a.y + o) = f4u{d[0], d[1], d[2], d[3]};
          if (a.z) *(f4u*)(a.z + o) = f4u{d[0], d[1], d[2], d[3]};
        } else {
          *(f2u*)(a.y + o) = f2u{d[0], d[1]};
          a.y[o + 2] = d[2];
          if (a.z) {
            *(f2u*)(a.z + o) = f2u{d[0], d[1]};
            a.z[o + 2] = d[2];
          }
        }
      }
    }
  }
}

int f7_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

bool fast_f32_w7_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M && !r.Tsub && r.w == F7_WS && r.layout == 0 &&
         r.H == F7_IW && r.W == F7_IW && r.oy == 0 && r.ox == 0 && r.B >= 1 && r.C >= 1;
}

// out: where the contraction's result goes (y, or the pre-mix map); out2: a second copy or null.
hipError_t launch_forward_fast_f32_w7(const FwdRequest& r, float* out, float* out2,
                                      hipStream_t st) {
  F7Args a{};
  a.B = r.B;
  a.C = r.C;
  a.items = (long long)r.B * r.C;
  a.x = (const float*)r.x;
  a.T = (const float*)r.T;
  a.y = out;
  a.z = out2;
  // persistent waves, 2 workgroups of 4 waves per CU, each wave at least one plane
  const long long cap = 2LL * f7_cu_count();
  const long long want = (a.items + 3) / 4;
  const int grid = (int)(want < cap ? want : cap);
  return launch_main(k_fwd_f32_w7, dim3(grid), dim3(256), 0, st, a);
}

}  // namespace wbmm
