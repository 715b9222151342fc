// repack.cpp -- host repack of the pages' weight formats into the T64 device
// images, and the inverse unpacks.  Pure byte and bit moves, no arithmetic.
//
// q8_row (cortiq-engine pages, q8_matvec_range: int8 [M][K] row-major,
// K % 4 == 0) -> T64: byte (o, i) at
//     ((o/64) * (Kp/16) + i/16) * 1024 + (o%64) * 16 + i%16.
//
// Q2 (qxmx qxmx_gpu.cpp page: dequant_embd, upload_q2, repack_q2_g64 /
// repack_q2_g128; blocks of an f16 d then group/4 code bytes, code k at bits
// 2*(k%4) of byte k/4) -> two T64 planes:
//   codes  [Mp/64][K/64][64][16 B]; in a unit's 16 bytes, weight
//          16j + 4a + b (j, a, b in 0..3) sits at bits 8b + 2a of
//          little-endian word j;
//   scales [Mp/64][K/group][64] binary16, copied bit for bit.
// Like upload_q2 on that page, rows are padded to a whole tile with zero
// codes and zero scales so that the kernels never read past the image.
#include <string.h>

#include <thread>
#include <vector>

#include "qg_internal.h"

namespace {

using qg::round_up;

bool q8_shape_ok(int64_t M, int64_t K) { return M >= 1 && K >= 4 && K % 4 == 0 && K <= (1 << 30) && M <= (1LL << 31) - 64; }

bool q2_shape_ok(int64_t M, int64_t K, int group) {
  return M >= 1 && (group == 64 || group == 128) && K >= group && K % group == 0 && K <= (1 << 30) &&
         M <= (1LL << 31) - 64;
}

// Runs f(t0, t1) over [0, n) in a few host threads (repack of ~1 GB images).
template <class F>
void parallel_tiles(int64_t n, F f) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = hw ? (hw > 16 ? 16 : hw) : 1;
  if (n < 64 || nt <= 1) {
    f(0, n);
    return;
  }
  if (nt > n) nt = n;
  std::vector<std::thread> th;
  for (int64_t t = 0; t < nt; t++) {
    int64_t a = n * t / nt, b = n * (t + 1) / nt;
    th.emplace_back([=] { f(a, b); });
  }
  for (auto &x : th) x.join();
}

// Bit transposition of one 64-weight unit.  src: 16 bytes, code k at bits
// 2*(k%4) of byte k/4.  dst: 16 bytes, weight 16j+4a+b at bit 8b+2a of
// little-endian word j.
inline void unit_to_t64(const uint8_t *src, uint8_t *dst) {
  for (int j = 0; j < 4; j++) {
    uint32_t w = 0;
    for (int a = 0; a < 4; a++)
      for (int b = 0; b < 4; b++) {
        const int k = 16 * j + 4 * a + b;
        const uint32_t code = (src[k >> 2] >> (2 * (k & 3))) & 3u;
        w |= code << (8 * b + 2 * a);
      }
    memcpy(dst + 4 * j, &w, 4);
  }
}

inline void unit_from_t64(const uint8_t *src, uint8_t *dst) {
  memset(dst, 0, 16);
  for (int j = 0; j < 4; j++) {
    uint32_t w;
    memcpy(&w, src + 4 * j, 4);
    for (int a = 0; a < 4; a++)
      for (int b = 0; b < 4; b++) {
        const int k = 16 * j + 4 * a + b;
        const uint32_t code = (w >> (8 * b + 2 * a)) & 3u;
        dst[k >> 2] |= (uint8_t)(code << (2 * (k & 3)));
      }
  }
}

}  // namespace

extern "C" {

size_t qg_q8row_packed_bytes(int64_t M, int64_t K) {
  if (!q8_shape_ok(M, K)) return 0;
  return (size_t)round_up(M, qg::kTileRows) * (size_t)round_up(K, qg::kQ8Chunk);
}

qg_status qg_repack_q8row(const int8_t *q, int64_t M, int64_t K, void *dst, size_t dst_bytes) {
  if (!q || !dst) return qg::fail(QG_EINVAL, "qg_repack_q8row: null pointer");
  if (!q8_shape_ok(M, K)) return qg::fail(QG_EINVAL, "qg_repack_q8row: bad shape M=%lld K=%lld (need M>=1, K>=4, K%%4==0)", (long long)M, (long long)K);
  const size_t need = qg_q8row_packed_bytes(M, K);
  if (dst_bytes < need) return qg::fail(QG_EINVAL, "qg_repack_q8row: dst_bytes %zu < %zu", dst_bytes, need);
  const int64_t tiles = round_up(M, 64) / 64, nchunk = round_up(K, 16) / 16;
  uint8_t *d = static_cast<uint8_t *>(dst);
  parallel_tiles(tiles, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; t++)
      for (int64_t c = 0; c < nchunk; c++)
        for (int r = 0; r < 64; r++) {
          uint8_t *o = d + ((t * nchunk + c) * 64 + r) * 16;
          const int64_t row = t * 64 + r;
          const int64_t k0 = c * 16;
          const int64_t n = row < M ? (K - k0 < 16 ? K - k0 : 16) : 0;
          if (n > 0) memcpy(o, q + row * K + k0, (size_t)n);
          if (n < 16) memset(o + n, 0, (size_t)(16 - n));
        }
  });
  return QG_OK;
}

qg_status qg_unpack_q8row(const void *packed, size_t packed_bytes, int64_t M, int64_t K, int8_t *q) {
  if (!packed || !q) return qg::fail(QG_EINVAL, "qg_unpack_q8row: null pointer");
  if (!q8_shape_ok(M, K)) return qg::fail(QG_EINVAL, "qg_unpack_q8row: bad shape");
  if (packed_bytes < qg_q8row_packed_bytes(M, K)) return qg::fail(QG_EINVAL, "qg_unpack_q8row: packed image too small");
  const int64_t nchunk = round_up(K, 16) / 16;
  const uint8_t *s = static_cast<const uint8_t *>(packed);
  for (int64_t row = 0; row < M; row++)
    for (int64_t c = 0; c < nchunk; c++) {
      const int64_t k0 = c * 16, n = K - k0 < 16 ? K - k0 : 16;
      memcpy(q + row * K + k0, s + (((row / 64) * nchunk + c) * 64 + row % 64) * 16, (size_t)n);
    }
  return QG_OK;
}

size_t qg_q2_blocks_bytes(int64_t M, int64_t K, int group) {
  if (!q2_shape_ok(M, K, group)) return 0;
  return (size_t)M * (size_t)(K / group) * (size_t)(2 + group / 4);
}

size_t qg_q2_codes_bytes(int64_t M, int64_t K) {
  if (!q2_shape_ok(M, K, 64)) return 0;
  return (size_t)round_up(M, 64) * (size_t)(K / 4);
}

size_t qg_q2_scales_bytes(int64_t M, int64_t K, int group) {
  if (!q2_shape_ok(M, K, group)) return 0;
  return (size_t)round_up(M, 64) * (size_t)(K / group) * 2;
}

qg_status qg_repack_q2(const void *blocks, size_t src_bytes, int64_t M, int64_t K, int group,
                       void *codes, size_t codes_bytes, void *scales, size_t scales_bytes) {
  if (!blocks || !codes || !scales) return qg::fail(QG_EINVAL, "qg_repack_q2: null pointer");
  if (!q2_shape_ok(M, K, group))
    return qg::fail(QG_EINVAL, "qg_repack_q2: bad shape M=%lld K=%lld group=%d", (long long)M, (long long)K, group);
  if (src_bytes != qg_q2_blocks_bytes(M, K, group))
    return qg::fail(QG_EINVAL, "qg_repack_q2: src_bytes %zu != M*(K/group)*(2+group/4) = %zu", src_bytes,
                    qg_q2_blocks_bytes(M, K, group));
  if (codes_bytes < qg_q2_codes_bytes(M, K)) return qg::fail(QG_EINVAL, "qg_repack_q2: codes plane too small");
  if (scales_bytes < qg_q2_scales_bytes(M, K, group)) return qg::fail(QG_EINVAL, "qg_repack_q2: scales plane too small");
  const int64_t tiles = round_up(M, 64) / 64, ng = K / group, nu = K / 64, upg = group / 64;
  const int64_t bb = 2 + group / 4;
  const uint8_t *src = static_cast<const uint8_t *>(blocks);
  uint8_t *cd = static_cast<uint8_t *>(codes);
  uint16_t *sd = static_cast<uint16_t *>(scales);
  parallel_tiles(tiles, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; t++)
      for (int r = 0; r < 64; r++) {
        const int64_t row = t * 64 + r;
        for (int64_t g = 0; g < ng; g++) {
          uint16_t dbits = 0;
          const uint8_t *blk = row < M ? src + (row * ng + g) * bb : nullptr;
          if (blk) dbits = (uint16_t)(blk[0] | (blk[1] << 8));
          sd[(t * ng + g) * 64 + r] = dbits;
          for (int64_t v = 0; v < upg; v++) {
            uint8_t *o = cd + ((t * nu + g * upg + v) * 64 + r) * 16;
            if (blk)
              unit_to_t64(blk + 2 + v * 16, o);
            else
              memset(o, 0, 16);
          }
        }
      }
  });
  return QG_OK;
}

qg_status qg_unpack_q2(const void *codes, size_t codes_bytes, const void *scales, size_t scales_bytes,
                       int64_t M, int64_t K, int group, void *blocks, size_t blocks_bytes) {
  if (!codes || !scales || !blocks) return qg::fail(QG_EINVAL, "qg_unpack_q2: null pointer");
  if (!q2_shape_ok(M, K, group)) return qg::fail(QG_EINVAL, "qg_unpack_q2: bad shape");
  if (codes_bytes < qg_q2_codes_bytes(M, K) || scales_bytes < qg_q2_scales_bytes(M, K, group) ||
      blocks_bytes < qg_q2_blocks_bytes(M, K, group))
    return qg::fail(QG_EINVAL, "qg_unpack_q2: buffer too small");
  const int64_t ng = K / group, nu = K / 64, upg = group / 64, bb = 2 + group / 4;
  const uint8_t *cs = static_cast<const uint8_t *>(codes);
  const uint16_t *ss = static_cast<const uint16_t *>(scales);
  uint8_t *dst = static_cast<uint8_t *>(blocks);
  for (int64_t row = 0; row < M; row++) {
    const int64_t t = row / 64, r = row % 64;
    for (int64_t g = 0; g < ng; g++) {
      uint8_t *blk = dst + (row * ng + g) * bb;
      const uint16_t dbits = ss[(t * ng + g) * 64 + r];
      blk[0] = (uint8_t)(dbits & 0xff);
      blk[1] = (uint8_t)(dbits >> 8);
      for (int64_t v = 0; v < upg; v++) unit_from_t64(cs + ((t * nu + g * upg + v) * 64 + r) * 16, blk + 2 + v * 16);
    }
  }
  return QG_OK;
}

}  // extern "C"
