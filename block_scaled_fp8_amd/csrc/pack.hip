// Offline weight preparation: row-major FP8 matrices -> tile-coalesced layout.
//
// Source: "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for
// Trainium2", file table: moe_w8.py prepares the expert weights offline and
// packs coalesced operands for the kernel.  The layout here is this library's
// own: for tile t (16 rows), 64-wide K chunk c and lane l, the 16 bytes a lane
// consumes are stored contiguously, so a wave's load of one tile chunk is a
// single 1 KB burst (see tile_lane_ptr).
#include "common.hpp"
#include "plan.hpp"

namespace moe {

// One thread moves one 16-byte piece; destination pieces are written in order.
__global__ __launch_bounds__(256) void pack_w8_kernel(const uint8_t* __restrict__ src,
                                                      uint8_t* __restrict__ dst, int64_t pieces,
                                                      int rows, int cols) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= pieces) return;
    const int64_t per_mat = (int64_t)rows * cols / 16;
    const int64_t mat = q / per_mat;
    int64_t r = q - mat * per_mat;
    const int lane = (int)(r & 63);
    r >>= 6;
    const int nch = cols / 64;
    const int c = (int)(r % nch);
    const int t = (int)(r / nch);
    const int row = 16 * t + (lane & 15);
    const int col = 64 * c + 16 * (lane >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + mat * rows * (int64_t)cols +
                                                    (int64_t)row * cols + col);
    *reinterpret_cast<u32x4*>(dst + q * 16) = v;
}

int launch_pack_w8(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                   hipStream_t stream) {
    const int64_t pieces = n_mats * (int64_t)rows * cols / 16;
    const int64_t blocks = (pieces + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) {
        set_error("moe_pack_w8: too many bytes in one call");
        return MOE_EINVAL;
    }
    prof_begin("pack_w8", stream);
    pack_w8_kernel<<<(unsigned)blocks, 256, 0, stream>>>(src, dst, pieces, rows, cols);
    prof_end(stream);
    return check_launch("pack_w8_kernel");
}

// MXFP4 scales for the tiled layout: for matrices [rows, cols] of E8M0 bytes
// (cols = K / 32), the byte lane l of a wave consumes for 16-row tile t and
// 128-wide K chunk c, S[16t + l%16][4c + l/16], is stored at (t * cols/4 + c)
// * 64 + l, so a wave's scale load of one tile chunk is one 64-byte line.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst,
                                                             int64_t n, int rows, int cols) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n) return;
    const int64_t per_mat = (int64_t)rows * cols;
    const int64_t mat = q / per_mat;
    int64_t r = q - mat * per_mat;
    const int lane = (int)(r & 63);
    r >>= 6;
    const int nch = cols / 4;
    const int c = (int)(r % nch);
    const int t = (int)(r / nch);
    dst[q] = src[mat * per_mat + (int64_t)(16 * t + (lane & 15)) * cols + 4 * c + (lane >> 4)];
}

int launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                          hipStream_t stream) {
    const int64_t n = n_mats * (int64_t)rows * cols;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) {
        set_error("moe_pack_mx_scales: too many bytes in one call");
        return MOE_EINVAL;
    }
    pack_mx_scales_kernel<<<(unsigned)blocks, 256, 0, stream>>>(src, dst, n, rows, cols);
    return check_launch("pack_mx_scales_kernel");
}

}  // namespace moe
