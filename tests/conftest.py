import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# A planted oracle mistake for the mutation check (CPU only): the oracle's
# pin tests run with it installed and must fail.
_MUTANT = os.environ.get("ZS3_ORACLE_MUTANT")
if _MUTANT:
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from hypothesis import Phase, settings as _hyp_settings

    _hyp_settings.register_profile("mutant", derandomize=True, deadline=None,
                                   phases=[Phase.explicit, Phase.reuse, Phase.generate])
    _hyp_settings.load_profile("mutant")
    import oracle_mutants

    oracle_mutants.install(_MUTANT)
