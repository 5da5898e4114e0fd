// Host driver for tests/test_dispatch_host.py: reads "M N K cus" lines and
// prints the GEMM kernel the dispatch rules choose for each, with its
// template arguments or tile.
#include <stdio.h>

#include "../int8_w8a8_quantized_token_amd/csrc/gemm_dispatch.h"

int main() {
  long long M, N, K, cus;
  while (scanf("%lld %lld %lld %lld", &M, &N, &K, &cus) == 4) {
    using namespace w8a8::dispatch;
    switch (gemm_path(M, N, K)) {
      case GemmPath::kMid: {
        const MidConfig m = mid_config(M, N, K, cus);
        printf("mid %d %d %d %d\n", m.mt, m.rw, m.nw, m.ns);
        break;
      }
      case GemmPath::kSkinny: {
        const SkinnyConfig k = skinny_config(M, N, K);
        printf("skinny %d %d %d %d %d\n", k.mt, k.rw, k.nw, k.u, k.late ? 1 : 0);
        break;
      }
      case GemmPath::kPrefill128: {
        const PrefillTile t = prefill_tile(M, N, cus);
        printf("prefill %s\n", t == PrefillTile::k256x192   ? "256x192"
                               : t == PrefillTile::k192x256 ? "192x256"
                                                            : "256x256");
        break;
      }
      case GemmPath::kPrefill64:
        printf("prefill64\n");
        break;
      case GemmPath::kTiled:
        printf("tiled\n");
        break;
    }
  }
  return 0;
}
