// temporary: GSA entry points not yet implemented
#include "../../include/gla.h"
extern "C" {
size_t gsa_fwd_workspace_bytes(int, int, int, int, int, int, int, int) { return 0; }
int gsa_fwd(const void*, const void*, const void*, const void*, const float*, const float*, void*, float*, float*,
            int, int, int, int, int, int, int, int, void*, size_t, void*) { return GLA_ERR_UNSUPPORTED; }
size_t gsa_bwd_workspace_bytes(int, int, int, int, int, int, int, int) { return 0; }
int gsa_bwd(const void*, const void*, const void*, const void*, const float*, const float*, const void*,
            const float*, const float*, void*, void*, void*, float*, float*, float*, int, int, int, int, int,
            int, int, int, void*, size_t, void*) { return GLA_ERR_UNSUPPORTED; }
}
