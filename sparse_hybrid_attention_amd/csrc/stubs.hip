#include "common.h"
using namespace shattn;
extern "C" size_t csa_index_topk_workspace_size(int, int, int, int, int, int) { return 0; }
extern "C" int csa_index_topk(const void*, const void*, const float*, int32_t*, int, int, int, int, int, int64_t, int, int, int, int, void*, size_t, void*) { return fail(SHATTN_EUNSUPPORTED, "not built"); }
