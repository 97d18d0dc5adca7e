// Host-side checks of container images (files and host buffers): the header
// against the layout, the scale / heavy-tailed / zero-nibble ranges, and the
// mask and perm sections.  Plain host code with no device calls, so a CPU test
// builds it with the address and undefined-behaviour sanitizers and feeds it
// malformed images.
#include <string.h>

#include "../../include/spectra.h"
#include "spectra_internal.h"

namespace spectra {

int check_shape(int64_t K, int64_t N) {
  if (K < 1 || K > SPECTRA_MAX_K) return fail(SPECTRA_E_INVAL, "K out of range [1, 2^24]");
  if (N < 1 || N > SPECTRA_MAX_N) return fail(SPECTRA_E_INVAL, "N out of range [1, 2^31]");
  // Keep every flat index and byte offset comfortably inside 63 bits and the
  // 1-D grids of the packing kernels inside their limits.
  if ((double)K * (double)N > (double)(1ull << 40))
    return fail(SPECTRA_E_INVAL, "N*K above 2^40 elements");
  return SPECTRA_OK;
}

namespace {
uint64_t rd64(const unsigned char* p) {
  uint64_t v;
  memcpy(&v, p, 8);
  return v;
}
}  // namespace

int parse_header(const unsigned char* h, uint64_t bytes, ImageFields& f) {
  if (bytes < kHeaderBytes) return fail(SPECTRA_E_INVAL, "image shorter than its 128-byte header");
  const uint64_t w0 = rd64(h);
  if ((uint32_t)w0 != kMagic) return fail(SPECTRA_E_INVAL, "bad magic");
  if ((uint32_t)(w0 >> 32) != kVersion) return fail(SPECTRA_E_INVAL, "unsupported version");
  f.K = (int64_t)rd64(h + 8);
  f.N = (int64_t)rd64(h + 16);
  f.K_b = (int64_t)rd64(h + 24);
  f.G = (int64_t)rd64(h + 32);
  f.n_out = (int64_t)rd64(h + 40);
  if (check_shape(f.K, f.N) != SPECTRA_OK) return SPECTRA_E_INVAL;
  if (f.n_out < 0 || f.n_out > f.K) return fail(SPECTRA_E_INVAL, "n_out out of range [0, K]");
  if (f.K_b != f.K - f.n_out) return fail(SPECTRA_E_INVAL, "K_b != K - n_out");
  if (f.G != (f.K_b + kGroup - 1) / kGroup) return fail(SPECTRA_E_INVAL, "G != ceil(K_b / 32)");
  f.lay = make_layout(f.K, f.N, f.n_out);
  const uint64_t want[7] = {f.lay.mask, f.lay.perm, f.lay.codes, f.lay.scales,
                            f.lay.zeros, f.lay.outliers, f.lay.total};
  for (int i = 0; i < 7; ++i)
    if (rd64(h + 48 + 8 * i) != want[i]) return fail(SPECTRA_E_INVAL, "section offsets differ from the layout");
  if (bytes != f.lay.total) return fail(SPECTRA_E_INVAL, "image size differs from total_bytes");
  return SPECTRA_OK;
}

int check_range(const ImageFields& f, uint64_t pos, const unsigned char* p, uint64_t len) {
  const uint64_t NG = (uint64_t)f.N * (uint64_t)f.G;
  auto overlap = [&](uint64_t a, uint64_t b, uint64_t& lo, uint64_t& hi) {
    lo = a > pos ? a : pos;
    hi = b < pos + len ? b : pos + len;
    return lo < hi;
  };
  uint64_t lo, hi;
  if (overlap(f.lay.scales, f.lay.scales + 2 * NG, lo, hi)) {
    for (uint64_t b = lo; b < hi; b += 2) {
      uint16_t h;
      memcpy(&h, p + (b - pos), 2);
      if ((h & 0x8000u) || (h & 0x7C00u) == 0x7C00u)
        return fail(SPECTRA_E_INVAL, "a scale is negative or not finite");
    }
  }
  const uint64_t ob = 2ull * (uint64_t)f.N * (uint64_t)f.n_out;
  if (overlap(f.lay.outliers, f.lay.outliers + ob, lo, hi)) {
    for (uint64_t b = lo; b < hi; b += 2) {
      uint16_t h;
      memcpy(&h, p + (b - pos), 2);
      if ((h & 0x7C00u) == 0x7C00u) return fail(SPECTRA_E_INVAL, "a heavy-tailed weight is not finite");
    }
  }
  if (NG & 1) {
    const uint64_t last = f.lay.zeros + NG / 2;  // byte holding the final nibble
    if (last >= pos && last < pos + len && (p[last - pos] >> 4) != 0)
      return fail(SPECTRA_E_INVAL, "the unused zero nibble is not 0");
  }
  return SPECTRA_OK;
}

// perm must be the bulk channels ascending, then the heavy-tailed ones
// ascending (the only order the packer writes).
int check_meta(const ImageFields& f, const uint32_t* mask, const int32_t* perm) {
  const int64_t words = (f.K + 31) / 32;
  int64_t set = 0;
  for (int64_t w = 0; w < words; ++w) {
    uint32_t m = mask[w];
    if (w == words - 1 && (f.K & 31)) {
      if (m >> (f.K & 31)) return fail(SPECTRA_E_INVAL, "mask bits set past K");
    }
    set += __builtin_popcount(m);
  }
  if (set != f.n_out) return fail(SPECTRA_E_INVAL, "mask does not flag n_out channels");
  int64_t b = 0, o = f.K_b;
  for (int64_t k = 0; k < f.K; ++k) {
    const bool heavy = (mask[k >> 5] >> (k & 31)) & 1u;
    const int64_t at = heavy ? o++ : b++;
    if (perm[at] != (int32_t)k) return fail(SPECTRA_E_INVAL, "perm is not the canonical channel order");
  }
  return SPECTRA_OK;
}

int validate_host_image(const unsigned char* img, uint64_t bytes, ImageFields& f) {
  if (parse_header(img, bytes, f) != SPECTRA_OK) return SPECTRA_E_INVAL;
  if (check_range(f, 0, img, bytes) != SPECTRA_OK) return SPECTRA_E_INVAL;
  return check_meta(f, reinterpret_cast<const uint32_t*>(img + f.lay.mask),
                    reinterpret_cast<const int32_t*>(img + f.lay.perm));
}

}  // namespace spectra
