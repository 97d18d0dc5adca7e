// Runs the library's host-side container-image checks (image.cpp) on image
// files, for a CPU test that builds both with the address and
// undefined-behaviour sanitizers.  Each file is read into a heap buffer of
// exactly its size, checked whole, then re-checked the way a streamed load
// does (header first, then ranges in chunks of the given sizes).  Prints one
// line per file: "<status whole> <status streamed>".
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "../include/spectra.h"
#include "../dequant_gemv_spectra_amd/csrc/spectra_internal.h"

namespace spectra {
// the harness's own error state (the library keeps its own in abi.hip)
static std::string g_msg;
void set_error(const std::string& msg, int) { g_msg = msg; }
int fail(int status, const std::string& msg) {
  g_msg = msg;
  return status;
}
}  // namespace spectra

int main(int argc, char** argv) {
  if (argc < 3) {
    fprintf(stderr, "usage: %s CHUNK FILE...\n", argv[0]);
    return 2;
  }
  const uint64_t chunk = strtoull(argv[1], nullptr, 10);
  for (int a = 2; a < argc; ++a) {
    FILE* fp = fopen(argv[a], "rb");
    if (!fp) return 3;
    fseek(fp, 0, SEEK_END);
    const long n = ftell(fp);
    fseek(fp, 0, SEEK_SET);
    unsigned char* buf = static_cast<unsigned char*>(malloc(n > 0 ? (size_t)n : 1));
    if (n > 0 && fread(buf, 1, (size_t)n, fp) != (size_t)n) return 4;
    fclose(fp);
    spectra::ImageFields f;
    const int whole = spectra::validate_host_image(buf, (uint64_t)n, f);
    // streamed: the header from its own 128-byte copy, then the ranges chunk
    // by chunk from exact-size copies, then mask and perm
    int streamed = SPECTRA_E_INVAL;
    if (n >= (long)spectra::kHeaderBytes) {
      unsigned char* hdr = static_cast<unsigned char*>(malloc(spectra::kHeaderBytes));
      memcpy(hdr, buf, spectra::kHeaderBytes);
      streamed = spectra::parse_header(hdr, (uint64_t)n, f);
      free(hdr);
      for (uint64_t pos = 0; streamed == SPECTRA_OK && pos < (uint64_t)n; pos += chunk) {
        const uint64_t len = (uint64_t)n - pos < chunk ? (uint64_t)n - pos : chunk;
        unsigned char* part = static_cast<unsigned char*>(malloc(len));
        memcpy(part, buf + pos, len);
        streamed = spectra::check_range(f, pos, part, len);
        free(part);
      }
      if (streamed == SPECTRA_OK)
        streamed = spectra::check_meta(f, reinterpret_cast<const uint32_t*>(buf + f.lay.mask),
                                       reinterpret_cast<const int32_t*>(buf + f.lay.perm));
    }
    printf("%d %d\n", whole, streamed);
    free(buf);
  }
  return 0;
}
