// Fast fp32 WBMM forward for w = 28 on NCHW 56x56 images (4 windows per image), table input:
// 784 x 784 per channel, so the work is bound by the fp32 matrix cores. The matrix is formed on
// chip from the table [gecl.asia reading notes, "Core Idea"; the notes' "Limitation" names the
// 28 x 28 window as the size where materializing M stops being practical].
//
// Persistent workgroups of 4 waves, two per CU, each walk a run of blocks of 32 windows (8 images)
// of one channel with v_mfma_f32_32x32x2f32 (32 output pixels x 32 windows x 2 K per instruction):
//   * output tiles are window rows: MFMA rows 0..27 are pixels 0..27 of the row, rows 28..31
//     pixels 24..27 again (their outputs are not stored); wave k owns rows 7k .. 7k+6, 7
//     accumulators of 16 registers;
//   * K is walked window row by window row; within a row, step s (0..13) takes pixel s for the
//     lower lane half and pixel s + 14 for the upper one;
//   * table operand: the (55, 55) table sits in LDS; M[(yi, xi)][(yk, xk)] =
//     T[yi - yk + 27][xi - xk + 27] is one LDS read at a per-lane base plus an immediate that
//     depends only on the tile, the K row and the step (every entry read is a real table entry);
//   * window operand: the block's K row (32 windows x 28 pixels) streams through a double-
//     buffered LDS row buffer, each lane's 14 pixels of a half row read as four 16-byte reads per
//     K row and shared by the wave's 7 tiles; one 16-byte global load per thread and row, issued
//     two rows ahead (across block boundaries);
//   * accumulators hold 4 consecutive pixels of a window row per lane: 16-byte stores. Images
//     past the batch read and write the batch's last image (same values), so no store or load
//     is predicated on the batch.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

#include <atomic>

namespace wbmm {
namespace {

constexpr int F28_WS = 28, F28_IW = 56, F28_PLANE = F28_IW * F28_IW;
constexpr int F28_L1 = 2 * F28_WS - 1, F28_L = F28_L1 * F28_L1;  // 55, 3025
constexpr int F28_NWB = 32;                 // windows per block
constexpr int F28_IPB = F28_NWB / 4;        // images per block
constexpr int F28_NT = F28_WS / 4;          // output row tiles per wave
constexpr int F28_XST = 36;                 // floats per window in a row buffer (two halves of
                                            // 14 at +0 and +16; 36 = 4 mod 32 spreads the banks)
constexpr int F28_XBUF = F28_NWB * F28_XST;
constexpr int F28_NLD = F28_NWB * 7;        // 16-byte pieces per K row (224)
constexpr int F28_TSZ = (F28_L + 3) / 4 * 4;
constexpr int f28_lds_bytes() { return (F28_TSZ + 2 * F28_XBUF) * 4; }

struct F28Args {
  int B, C, groups;  // groups: blocks per channel
  const float* x;
  const float* T;
  float* y;
  float* z;          // a second copy of the output, or null
};

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32_f32(float a, float b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_fwd_f32_w28(F28Args a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  float* Ts = smem_f;                  // [L] table
  float* xbuf = smem_f + F28_TSZ;      // [2][NWB][XST]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nb = a.C * a.groups;
  const int b0 = (int)((long long)blockIdx.x * nb / gridDim.x);
  const int b1 = (int)((long long)(blockIdx.x + 1) * nb / gridDim.x);
  if (b0 >= b1) return;  // uniform over the workgroup
  struct Blk {
    int c, img0, nimg;
  };
  auto blk = [&](int b) {
    Blk k;
    k.c = b / a.groups;
    k.img0 = (b - k.c * a.groups) * F28_IPB;
    k.nimg = min(a.B - k.img0, F28_IPB);
    return k;
  };
  // element offset of the plane of image im of block k (images past the batch: its last image)
  auto plane = [&](const Blk& k, int im) {
    return ((size_t)(k.img0 + min(im, k.nimg - 1)) * a.C + k.c) * F28_PLANE;
  };

  // row loads: thread t -> window jw = t / 7, pixels 4p .. 4p + 3 (p = t % 7); threads past the
  // 224 pieces load piece 223 again and do not write it
  const int tl = min((int)threadIdx.x, F28_NLD - 1);
  const int jw = tl / 7, pp = tl - (tl / 7) * 7;
  const bool writer = threadIdx.x < F28_NLD;
  const int ld_off = (F28_WS * ((jw >> 1) & 1)) * F28_IW + F28_WS * (jw & 1) + 4 * pp;
  // LDS places of the piece's two pixel pairs (pairs never straddle the half-row boundary)
  const int q0 = 4 * pp, q1 = 4 * pp + 2;
  const int st0 = jw * F28_XST + (q0 / 14) * 16 + q0 % 14;
  const int st1 = jw * F28_XST + (q1 / 14) * 16 + q1 % 14;
  auto ld_base = [&](const Blk& k) { return plane(k, jw >> 2) + ld_off; };
  auto load_row = [&](size_t base, int yk) {
    return *(const float4*)(a.x + base + (size_t)yk * F28_IW);
  };
  auto store_row = [&](const float4& v, int buf) {
    if (writer) {
      float* xb = xbuf + buf * F28_XBUF;
      *(float2*)(xb + st0) = make_float2(v.x, v.y);
      *(float2*)(xb + st1) = make_float2(v.z, v.w);
    }
  };
  // table: every thread loads its entries, then (after a barrier) writes them
  auto stage_table = [&](int c) {
    constexpr int NQ = (F28_L + 255) / 256;
    float tv[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = min((int)threadIdx.x + 256 * j, F28_L - 1);
      tv[j] = a.T[(size_t)c * F28_L + q];
    }
    __syncthreads();  // every wave is done with the previous table
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = threadIdx.x + 256 * j;
      if (q < F28_L) Ts[q] = tv[j];
    }
  };

  Blk cur = blk(b0);
  size_t base_cur = ld_base(cur);
  float4 pre[2];  // K row r of the stream in slot r % 2
  pre[0] = load_row(base_cur, 0);
  pre[1] = load_row(base_cur, 1);
  int table_c = cur.c;
  stage_table(cur.c);
  store_row(pre[0], 0);
  __syncthreads();

  // lane (l32, kh): MFMA row l32 = pixel slot, column l32 = window, K half kh
  const int l32 = lane & 31, kh = lane >> 5;
  const int xi = l32 < F28_WS ? l32 : l32 - 4;
  const int t0 = F28_NT * wave;  // first output window row of this wave
  // table index of tile t, K row yk, step s:
  //   (t0 + t - yk + 27) * 55 + xi + 27 - 14 kh - s = abase + (27 - yk) * 55 + (t * 55 + 13 - s)
  const int abase = t0 * F28_L1 + xi + 14 - 14 * kh;
  const int xb = l32 * F28_XST + 16 * kh;

  for (int b = b0; b < b1; ++b) {
    const Blk nxt = blk(b + 1 < b1 ? b + 1 : b);  // the last block's lookahead re-reads itself
    const size_t base_nxt = ld_base(nxt);
    if (cur.c != table_c) {  // uniform
      stage_table(cur.c);
      table_c = cur.c;
      __syncthreads();
    }
    v16f acc[F28_NT];
#pragma unroll
    for (int t = 0; t < F28_NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
    // K rows in pairs (row yk in slot and buffer yk % 2); row yk + 2 of the stream goes in
    // flight into the slot row yk has left, row yk + 1 goes to the other buffer at the end
    for (int yk0 = 0; yk0 < F28_WS; yk0 += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int yk = yk0 + h;
        const int yn = yk + 2;
        pre[h] = yn < F28_WS ? load_row(base_cur, yn) : load_row(base_nxt, yn - F28_WS);
        const float* xs = xbuf + h * F28_XBUF + xb;
        float bv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = *(const float4*)(xs + 4 * i);
          bv[4 * i] = v.x;
          bv[4 * i + 1] = v.y;
          bv[4 * i + 2] = v.z;
          bv[4 * i + 3] = v.w;
        }
        const float* ap = Ts + abase + (F28_WS - 1 - yk) * F28_L1;
        float av[F28_NT], an[F28_NT];
#pragma unroll
        for (int t = 0; t < F28_NT; ++t) av[t] = ap[t * F28_L1 + 13];
#pragma unroll
        for (int s = 0; s < 14; ++s) {
          if (s + 1 < 14) {
#pragma unroll
            for (int t = 0; t < F28_NT; ++t) an[t] = ap[t * F28_L1 + 13 - (s + 1)];
          }
#pragma unroll
          for (int t = 0; t < F28_NT; ++t) acc[t] = mfma32_f32(av[t], bv[s], acc[t]);
          if (s + 1 < 14) {
#pragma unroll
            for (int t = 0; t < F28_NT; ++t) av[t] = an[t];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // row yk + 1 into the other buffer (every wave is past row yk - 1, which used it)
        store_row(pre[h ^ 1], h ^ 1);
        __syncthreads();
      }
    }
    // stores: lane (window l32, kh) holds slots 8g + 4kh .. + 3 of each tile's window row; slots
    // 28..31 (g = 3, kh = 1) repeat pixels 24..27 and are not stored
    {
      const int j = l32;
      const size_t ob = plane(cur, j >> 2) + (size_t)(F28_WS * ((j >> 1) & 1) + t0) * F28_IW +
                        F28_WS * (j & 1) + 4 * kh;
#pragma unroll
      for (int t = 0; t < F28_NT; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g == 3 && kh) continue;
          const float4 v = make_float4(acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2],
                                       acc[t][4 * g + 3]);
          const size_t o = ob + (size_t)t * F28_IW + 8 * g;
          *(float4*)(a.y + o) = v;
          if (a.z) *(float4*)(a.z + o) = v;
        }
      }
    }
    cur = nxt;
    base_cur = base_nxt;
  }
}

int f28_cu_count() {
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

bool fast_f32_w28_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M && !r.Tsub && r.w == F28_WS && r.layout == 0 &&
         r.H == F28_IW && r.W == F28_IW && r.oy == 0 && r.ox == 0 && r.B >= 1 && r.C >= 1 &&
         (long long)r.C * ((r.B + F28_IPB - 1) / F28_IPB) < (1LL << 31);
}

// out: where the contraction's result goes (y, or the pre-mix map); out2: a second copy or null.
hipError_t launch_forward_fast_f32_w28(const FwdRequest& r, float* out, float* out2,
                                       hipStream_t st) {
  F28Args a{};
  a.B = r.B;
  a.C = r.C;
  a.groups = (r.B + F28_IPB - 1) / F28_IPB;
  a.x = (const float*)r.x;
  a.T = (const float*)r.T;
  a.y = out;
  a.z = out2;
  const long long nb = (long long)a.C * a.groups;
  const long long cap = 2LL * f28_cu_count();
  const int grid = (int)(nb < cap ? nb : cap);
  hipError_t e = hipFuncSetAttribute((const void*)k_fwd_f32_w28,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, f28_lds_bytes());
  if (e != hipSuccess) return e;
  return launch_main(k_fwd_f32_w28, dim3(grid), dim3(256), f28_lds_bytes(), st, a);
}

}  // namespace wbmm
